// Output projection with the Δattn score fused into its epilogue.
//
// U = O · Wo^T (Wo stored out-major [hidden, Hq*D]) is the attention
// sublayer's update to the residual stream, and the token score is its row
// norm ||U_t||_2 — CSDN explainer "DASH：基于注意力增量的Transformer令牌压缩，
// 实现长序列推理高效加速", §2.1 (U and Δattn) and §2.2 (the norm costs next to
// nothing once U is produced).
//
// bf16 path: 256x256 output tile per 512-thread workgroup (8 waves of 64x128),
// K stepped by 64, operands streamed into a double-buffered LDS ring by direct
// global->LDS loads (no register staging) a whole step ahead of their use
// (v_mfma_f32_32x32x16_bf16, fp32 accumulation).  Inside a step the operand
// reads of each 16-wide k-step are issued between the MFMAs of the previous
// one in a fixed order, so two waves per SIMD keep the matrix unit fed; rows
// are XOR-swizzled so the operand reads are free of bank conflicts, and tiles
// are grouped so the workgroups running together share their A rows and W
// slices in L2.  The tile is computed transposed (C^T = Wo_tile · O_tile^T) so
// that every lane holds a single output row: the row's sum of squares is then
// accumulated in registers straight from the fp32 accumulators, before U is
// rounded to bf16.  Each (row, column tile) partial is written to the
// workspace and a finalize kernel adds the partials in a fixed order and takes
// the square root, so the score is bit-reproducible run to run (no atomics).
// A 224-column variant (below) is picked when it fills the chip better.
#include <atomic>
#include <type_traits>

#include "dash_common.h"
#include "dash_kernels.h"

namespace dash {

namespace {

constexpr int kGemmThreads = 512;                       // 8 waves
constexpr int kBM = 256;                                // rows of U (tokens) per tile
constexpr int kBN = 256;                                // columns of U (hidden channels) per tile
constexpr int kBK = 64;                                 // contraction step: one 128-byte LDS row
constexpr int kStages = 2;                              // LDS ring depth (loads run 1 step ahead)
constexpr int kRowBytes = kBK * 2;
constexpr int kRowChunks = kRowBytes / 16;              // 16-byte chunks per row
constexpr int kRowsPerLine = 256 / kRowBytes;           // rows sharing one 64-bank line
constexpr int kATileBytes = kBM * kRowBytes;            // 32 KiB
constexpr int kWTileBytes = kBN * kRowBytes;            // 32 KiB
constexpr int kStageBytes = kATileBytes + kWTileBytes;  // 64 KiB
constexpr int kGroupM = 4;                              // m-tiles per L2-sharing group
constexpr int kNB = 4;                                  // 32-column blocks per wave (128 columns)
constexpr int kMB = 2;                                  // 32-row blocks per wave (64 rows)

// Row r keeps its 16-byte chunk c at slot c ^ ((r / kRowsPerLine) % kRowChunks):
// the 16 lanes of one 16-byte operand read (16 consecutive rows) then hit
// distinct banks of the 64-bank LDS.
template <int RB = kRowBytes>
__device__ __forceinline__ int gemm_slot(int row, int chunk) {
  constexpr int kChunksT = RB / 16, kPerLineT = 256 / RB;
  return chunk ^ ((row / kPerLineT) % kChunksT);
}

// Buffer resource over `bytes` bytes from `base` (capped at the 32-bit range,
// which always covers one tile's rows): loads past the end return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t gemm_rsrc(const void* base, int64_t bytes) {
  const int n = static_cast<int>(bytes > 0xffffffffll ? 0xffffffffll : (bytes < 0 ? 0 : bytes));
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), n, 0x00020000);
}

// Global->LDS loads of one stage through buffer loads: the A and W tiles get a
// buffer resource each, starting at the tile's first row, so a lane's byte
// offset (row, swizzled chunk) is fixed and the k step rides in the scalar
// offset; rows past the matrix edge read zeros (their results are never
// stored).  The wave index is made uniform so the LDS destinations stay scalar.
template <int BN, int NW = kGemmThreads / 64, int RB = kRowBytes>
struct GemmLoadPlan {
  static constexpr int kABytes = kBM * RB;
  static constexpr int kWBytes = BN * RB;
  static constexpr int kStage = kABytes + kWBytes;
  static constexpr int kChunks = kStage / 1024;                              // 1 KiB per wave-wide load
  static constexpr int kPerWave = (kChunks + NW - 1) / NW;
  static_assert(kStage % 1024 == 0, "whole KiB per stage");
  __amdgpu_buffer_rsrc_t a_src, w_src;
  uint32_t voff[kPerWave];  // this lane's row and swizzled chunk, at k = 0
  __device__ __forceinline__ void init(const uint16_t* A, const uint16_t* W, int m0, int n0, int M, int N, int K) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    constexpr int kRowsPerKiB = 1024 / RB;
    constexpr int kChunksPerRow = RB / 16;
    a_src = gemm_rsrc(A + static_cast<size_t>(m0) * K, static_cast<int64_t>(M - m0) * K * 2);
    w_src = gemm_rsrc(W + static_cast<size_t>(n0) * K, static_cast<int64_t>(N - n0) * K * 2);
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
      const int q = min(wave + NW * i, kChunks - 1);  // 1 KiB chunk of the stage
      const int is_a = q < kABytes / 1024;
      const int local_row = (is_a ? q : q - kABytes / 1024) * kRowsPerKiB + lane / kChunksPerRow;
      const int chunk = gemm_slot<RB>(local_row, lane % kChunksPerRow);
      voff[i] = static_cast<uint32_t>(local_row) * static_cast<uint32_t>(K) * 2u + chunk * 16;
    }
  }
  __device__ __forceinline__ void issue(unsigned char* stage, int k0) const {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
      const int q = wave + NW * i;
      // A chunks come first and split evenly over the waves: load i of every
      // wave is an A chunk iff i < (A chunks) / NW
      static_assert((kABytes / 1024) % NW == 0, "A chunks split evenly over the waves");
      if (NW * (i + 1) <= kChunks || q < kChunks)  // only the last load can be missing (wave-uniform)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(i < kABytes / 1024 / NW ? a_src : w_src,
                                                 (__attribute__((address_space(3))) void*)(stage + q * 1024), 16,
                                                 voff[i], k0 * 2, 0, 0);
    }
  }
  // After two issue() calls: wait until this wave's loads of the first have
  // landed.  When the chunks do not split evenly, waves differ in how many
  // loads a stage takes, so they wait for both.
  __device__ __forceinline__ void wait_first_of_two() const {
    if constexpr (kChunks % NW == 0) {
      static_assert(kPerWave < 64, "vmcnt range");
      __builtin_amdgcn_s_waitcnt(0x0F70 | (kPerWave & 15) | ((kPerWave >> 4) << 14));
    } else {
      __builtin_amdgcn_s_waitcnt(0x0F70);
    }
  }
};

__device__ __forceinline__ void wait_vmcnt_0() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)
__device__ __forceinline__ void wait_lgkm_0() { __builtin_amdgcn_s_waitcnt(0xC07F); }   // lgkmcnt(0)

// Issue order inside one 16-wide k-step: one MFMA first, then the LDS reads
// of the next k-step (and, in the last k-step of a stage, the global->LDS
// loads of the stage after next) one between each pair of the remaining
// MFMAs, so that a read or load waiting for its unit does not hold up the
// matrix unit.  Masks: 0x008 MFMA, 0x020 VMEM read, 0x100 DS read.
template <bool kLoads, bool kReads>
__device__ __forceinline__ void gemm_ks_order() {
  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
#pragma unroll
  for (int i = 0; i < 6; ++i) {
    if (kReads) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    if (kLoads) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  }
  if (kLoads) __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);
  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
}

__global__ __launch_bounds__(kGemmThreads, 1)
void wo_gemm_bf16_kernel(const uint16_t* __restrict__ A, const uint16_t* __restrict__ W,
                         uint16_t* __restrict__ U, float* __restrict__ part,
                         const int32_t* __restrict__ m_dev, int M_max, int N, int K, int n_tiles_n,
                         int part_ld) {
  __shared__ __attribute__((aligned(1024))) unsigned char lds[kStages * kStageBytes];
  int M = m_dev ? *m_dev : M_max;
  if (M > M_max) M = M_max;
  const int n_tiles_m = (M_max + kBM - 1) / kBM;
  const int lid = xcd_remap_chunked(blockIdx.x, n_tiles_m * n_tiles_n, kGroupM * n_tiles_n);
  // Groups of kGroupM m-tiles sweep all n-tiles together (shared A rows and W
  // k-slices stay in L2 while the group runs).
  const int group = lid / (kGroupM * n_tiles_n);
  const int gm = min(kGroupM, n_tiles_m - group * kGroupM);
  const int within = lid - group * kGroupM * n_tiles_n;
  const int tm = group * kGroupM + within % gm;
  const int tn = within / gm;
  const int m0 = tm * kBM;
  const int n0 = tn * kBN;
  if (m0 >= M) return;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int wm = wave & 3;   // 64-row slice of the tile
  const int wn = wave >> 2;  // 128-column slice of the tile

  GemmLoadPlan<kBN> plan;
  plan.init(A, W, m0, n0, M, N, K);

  // Per-lane byte offsets of the 16-byte operand chunk for each 16-wide k-step.
  int koff[kBK / 16];
#pragma unroll
  for (int ks = 0; ks < kBK / 16; ++ks) koff[ks] = 16 * gemm_slot(l32, 2 * ks + hi);
  const int a_row = (wm * 64 + l32) * kRowBytes;                  // O rows (B operand)
  const int w_row = kATileBytes + (wn * 128 + l32) * kRowBytes;   // W rows (A operand)

  f32x16 acc[kNB][kMB];
#pragma unroll
  for (int i = 0; i < kNB; ++i)
#pragma unroll
    for (int j = 0; j < kMB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // The operands of 16-wide k-step ks+1 are read while step ks multiplies,
  // and step kt+1's first operands are read during step kt's last MFMAs.
  // Step kt+2 is loaded into step kt's stage as soon as every wave has read
  // step kt (the barrier in the last k-step), a whole step ahead of its use.
  // The last two steps are peeled off (no loads after them, no reads after
  // the last) so that every k-step's issue order is fixed at compile time.
  const int KT = K / kBK;
  auto stage = [&](int kt) { return lds + (kt & 1) * kStageBytes; };
  bf16x8 opw[2][kNB], opa[2][kMB];
  auto read_ks = [&](const unsigned char* st, int ks, int buf) {
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb)
      opw[buf][nb] = *reinterpret_cast<const bf16x8*>(st + w_row + nb * 32 * kRowBytes + koff[ks]);
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb)
      opa[buf][mb] = *reinterpret_cast<const bf16x8*>(st + a_row + mb * 32 * kRowBytes + koff[ks]);
  };
  auto step = [&](int kt, auto loads_c, auto next_c) {
    constexpr bool kLoadNext = decltype(loads_c)::value;  // kt + 2 < KT
    constexpr bool kHasNext = decltype(next_c)::value;    // kt + 1 < KT
    const unsigned char* st = stage(kt);
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      const int cur = ks & 1;
      if (ks + 1 < kBK / 16) {
        read_ks(st, ks + 1, cur ^ 1);
      } else {
        wait_lgkm_0();                 // this wave's reads of step kt are done
        wait_vmcnt_0();                // its part of step kt+1 has landed
        __builtin_amdgcn_s_barrier();  // ... and every wave's; no wave reads stage kt any more
        __builtin_amdgcn_sched_barrier(0);
        if (kLoadNext) plan.issue(stage(kt), (kt + 2) * kBK);
        if (kHasNext) read_ks(stage(kt + 1), 0, cur ^ 1);
      }
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb)
#pragma unroll
        for (int mb = 0; mb < kMB; ++mb) acc[nb][mb] = mfma32x32x16(opw[cur][nb], opa[cur][mb], acc[nb][mb]);
      if (ks + 1 < kBK / 16)
        gemm_ks_order<false, true>();
      else
        gemm_ks_order<kLoadNext, kHasNext>();
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  plan.issue(stage(0), 0);
  if (KT > 1) {
    plan.issue(stage(1), kBK);
    plan.wait_first_of_two();
  } else {
    wait_vmcnt_0();
  }
  __builtin_amdgcn_s_barrier();
  read_ks(stage(0), 0, 0);
  __builtin_amdgcn_sched_barrier(0);
  int kt = 0;
  for (; kt + 2 < KT; ++kt) step(kt, std::true_type{}, std::true_type{});
  if (kt + 1 < KT) step(kt++, std::false_type{}, std::true_type{});
  if (kt < KT) step(kt, std::false_type{}, std::false_type{});

  // ---- epilogue -----------------------------------------------------------
  // acc[nb][mb][r] = U[m][n] with m = m0 + wm*64 + mb*32 + l32,
  //                  n = n0 + wn*128 + nb*32 + (r/4)*8 + hi*4 + (r%4).
  wait_lgkm_0();
  __builtin_amdgcn_s_barrier();  // every wave is done with the ring before it is reused
  float* red = reinterpret_cast<float*>(lds);                // [2 wn][256 m] partial sums
  uint16_t* ct = reinterpret_cast<uint16_t*>(lds + 4096);    // staging [128 m][kLdsC], one half at a time
  constexpr int kLdsC = kBN + 8;
  if (part) {  // the score's partial sums only when the score is asked for
    const bool full = n0 + kBN <= N;  // no column of the tile past the matrix edge
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb) {
      float ss = 0.f;
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int nl = wn * 128 + nb * 32 + (r >> 2) * 8 + hi * 4 + (r & 3);
          const float v = (full || n0 + nl < N) ? acc[nb][mb][r] : 0.f;
          ss += v * v;
        }
      ss += __shfl_xor(ss, 32, 64);
      if (hi == 0) red[wn * kBM + wm * 64 + mb * 32 + l32] = ss;
    }
  }
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    if ((wm >> 1) == half) {
#pragma unroll
      for (int mb = 0; mb < kMB; ++mb) {
        const int ml = (wm & 1) * 64 + mb * 32 + l32;  // row within this half
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int nl = wn * 128 + nb * 32 + g * 8 + hi * 4;
            u32x2 pk;
            pk[0] = pack_bf16x2(acc[nb][mb][g * 4 + 0], acc[nb][mb][g * 4 + 1]);
            pk[1] = pack_bf16x2(acc[nb][mb][g * 4 + 2], acc[nb][mb][g * 4 + 3]);
            *reinterpret_cast<u32x2*>(ct + ml * kLdsC + nl) = pk;
          }
      }
    }
    __syncthreads();
    // Coalesced store of 128 rows x 32 chunks of 16 bytes.
#pragma unroll
    for (int i = 0; i < (128 * kBN / 8) / kGemmThreads; ++i) {
      const int c = tid + i * kGemmThreads;
      const int row = c >> 5;
      const int cc = c & 31;
      const int m = m0 + half * 128 + row;
      const int n = n0 + cc * 8;
      if (m < M && n < N) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(ct + row * kLdsC + cc * 8);
        if (n + 8 <= N) {
          *reinterpret_cast<u32x4*>(U + static_cast<size_t>(m) * N + n) = v;
        } else {
          for (int j = 0; j < N - n; ++j)
            U[static_cast<size_t>(m) * N + n + j] = static_cast<uint16_t>(v[j >> 1] >> (16 * (j & 1)));
        }
      }
    }
    __syncthreads();
  }
  if (part && tid < kBM) {
    const int m = m0 + tid;
    if (m < M) part[static_cast<size_t>(tn) * part_ld + m] = red[tid] + red[kBM + tid];
  }
}

// ---------------------------------------------------------------------------
// bf16 path with 224-column tiles.  Same ring, loads and swizzle as above; the
// 8 waves split the 256x224 tile as 4 (tokens) x 2 (channels), 64 x 112 each,
// which is 4 x 7 blocks of v_mfma_f32_16x16x32_bf16.  224 divides the hidden
// width 3584 (Qwen2.5-7B), so row counts that are multiples of 256 fill whole
// waves of 256 workgroups where 256-column tiles leave part of the chip idle.
// ---------------------------------------------------------------------------
constexpr int kBN224 = 224;
constexpr int kStage224 = kATileBytes + kBN224 * kRowBytes;  // 60 KiB
constexpr int kTB = 4;  // 16-token blocks per wave (64 tokens)
constexpr int kCB = 7;  // 16-channel blocks per wave (112 channels)

// Issue order of one 32-wide k-step of the 224-column kernel (28 MFMAs of
// 16x16x32, 11 operand reads, up to 8 loads in the last k-step of a stage).
template <bool kLoads, bool kReads>
__device__ __forceinline__ void gemm224_ks_order() {
  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
#pragma unroll
  for (int i = 0; i < 11; ++i) {
    if (kReads) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    if (kLoads && i < 8) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 5, 0);
}

__global__ __launch_bounds__(kGemmThreads, 1)
void wo_gemm_bf16_n224_kernel(const uint16_t* __restrict__ A, const uint16_t* __restrict__ W,
                              uint16_t* __restrict__ U, float* __restrict__ part,
                              const int32_t* __restrict__ m_dev, int M_max, int N, int K, int n_tiles_n,
                              int part_ld) {
  __shared__ __attribute__((aligned(1024))) unsigned char lds[kStages * kStage224];
  int M = m_dev ? *m_dev : M_max;
  if (M > M_max) M = M_max;
  const int n_tiles_m = (M_max + kBM - 1) / kBM;
  const int lid = xcd_remap_chunked(blockIdx.x, n_tiles_m * n_tiles_n, kGroupM * n_tiles_n);
  const int group = lid / (kGroupM * n_tiles_n);
  const int gm = min(kGroupM, n_tiles_m - group * kGroupM);
  const int within = lid - group * kGroupM * n_tiles_n;
  const int tm = group * kGroupM + within % gm;
  const int tn = within / gm;
  const int m0 = tm * kBM;
  const int n0 = tn * kBN224;
  if (m0 >= M) return;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l16 = lane & 15;
  const int q4 = lane >> 4;  // which 8-wide k slice of a 32-wide step this lane supplies
  const int wm = wave & 3;   // 64-token slice of the tile
  const int wn = wave >> 2;  // 112-channel slice of the tile

  GemmLoadPlan<kBN224> plan;
  plan.init(A, W, m0, n0, M, N, K);

  // Operand rows start at multiples of 16, so a lane's swizzled chunk offset
  // depends only on l16 and the k step.
  int koff[kBK / 32];
#pragma unroll
  for (int ks = 0; ks < kBK / 32; ++ks) koff[ks] = 16 * gemm_slot(l16, 4 * ks + q4);
  const int a_row = (wm * 64 + l16) * kRowBytes;                   // O rows (B operand)
  const int w_row = kATileBytes + (wn * 112 + l16) * kRowBytes;    // W rows (A operand)

  f32x4 acc[kCB][kTB];
#pragma unroll
  for (int i = 0; i < kCB; ++i)
#pragma unroll
    for (int j = 0; j < kTB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Same pipeline as the 256-column kernel, in 32-wide k-steps: the
  // operands of the second half of a stage are read while the first half
  // multiplies, and the next stage's first operands while the second does.
  const int KT = K / kBK;
  auto stage = [&](int kt) { return lds + (kt & 1) * kStage224; };
  bf16x8 opw[2][kCB], opa[2][kTB];
  auto read_ks = [&](const unsigned char* st, int ks, int buf) {
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb)
      opw[buf][cb] = *reinterpret_cast<const bf16x8*>(st + w_row + cb * 16 * kRowBytes + koff[ks]);
#pragma unroll
    for (int tb = 0; tb < kTB; ++tb)
      opa[buf][tb] = *reinterpret_cast<const bf16x8*>(st + a_row + tb * 16 * kRowBytes + koff[ks]);
  };
  auto step = [&](int kt, auto loads_c, auto next_c) {
    constexpr bool kLoadNext = decltype(loads_c)::value;  // kt + 2 < KT
    constexpr bool kHasNext = decltype(next_c)::value;    // kt + 1 < KT
    const unsigned char* st = stage(kt);
#pragma unroll
    for (int ks = 0; ks < kBK / 32; ++ks) {
      const int cur = ks & 1;
      if (ks + 1 < kBK / 32) {
        read_ks(st, ks + 1, cur ^ 1);
      } else {
        wait_lgkm_0();
        wait_vmcnt_0();
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        if (kLoadNext) plan.issue(stage(kt), (kt + 2) * kBK);
        if (kHasNext) read_ks(stage(kt + 1), 0, cur ^ 1);
      }
#pragma unroll
      for (int cb = 0; cb < kCB; ++cb)
#pragma unroll
        for (int tb = 0; tb < kTB; ++tb) acc[cb][tb] = mfma16x16x32(opw[cur][cb], opa[cur][tb], acc[cb][tb]);
      if (ks + 1 < kBK / 32)
        gemm224_ks_order<false, true>();
      else
        gemm224_ks_order<kLoadNext, kHasNext>();
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  plan.issue(stage(0), 0);
  if (KT > 1) {
    plan.issue(stage(1), kBK);
    plan.wait_first_of_two();
  } else {
    wait_vmcnt_0();
  }
  __builtin_amdgcn_s_barrier();
  read_ks(stage(0), 0, 0);
  __builtin_amdgcn_sched_barrier(0);
  int kt = 0;
  for (; kt + 2 < KT; ++kt) step(kt, std::true_type{}, std::true_type{});
  if (kt + 1 < KT) step(kt++, std::false_type{}, std::true_type{});
  if (kt < KT) step(kt, std::false_type{}, std::false_type{});

  // ---- epilogue -----------------------------------------------------------
  // acc[cb][tb][r] = U[m][n] with m = m0 + wm*64 + tb*16 + l16,
  //                  n = n0 + wn*112 + cb*16 + q4*4 + r.
  wait_lgkm_0();
  __builtin_amdgcn_s_barrier();
  float* red = reinterpret_cast<float*>(lds);              // [2 wn][256 m] partial sums
  uint16_t* ct = reinterpret_cast<uint16_t*>(lds + 4096);  // staging [256 m][kLdsC]
  constexpr int kLdsC = kBN224 + 8;
  static_assert(4096 + kBM * kLdsC * 2 <= kStages * kStage224, "staging fits the ring");
  const bool full = n0 + kBN224 <= N;  // no column of the tile past the matrix edge
#pragma unroll
  for (int tb = 0; tb < kTB; ++tb) {
    if (part) {  // the score's partial sums only when the score is asked for
      float ss = 0.f;
#pragma unroll
      for (int cb = 0; cb < kCB; ++cb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int nl = wn * 112 + cb * 16 + q4 * 4 + r;
          const float v = (full || n0 + nl < N) ? acc[cb][tb][r] : 0.f;
          ss += v * v;
        }
      ss += __shfl_xor(ss, 16, 64);
      ss += __shfl_xor(ss, 32, 64);
      if (q4 == 0) red[wn * kBM + wm * 64 + tb * 16 + l16] = ss;
    }
    const int ml = wm * 64 + tb * 16 + l16;
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb) {
      const int nl = wn * 112 + cb * 16 + q4 * 4;
      u32x2 pk;
      pk[0] = pack_bf16x2(acc[cb][tb][0], acc[cb][tb][1]);
      pk[1] = pack_bf16x2(acc[cb][tb][2], acc[cb][tb][3]);
      *reinterpret_cast<u32x2*>(ct + ml * kLdsC + nl) = pk;
    }
  }
  __syncthreads();
  // Coalesced store of 256 rows x 28 chunks of 16 bytes.
  constexpr int kChunksRow = kBN224 / 8;
#pragma unroll 2
  for (int i = 0; i < (kBM * kChunksRow) / kGemmThreads; ++i) {
    const int c = tid + i * kGemmThreads;
    const int row = c / kChunksRow;
    const int cc = c - row * kChunksRow;
    const int m = m0 + row;
    const int n = n0 + cc * 8;
    if (m < M && n < N) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(ct + row * kLdsC + cc * 8);
      if (n + 8 <= N) {
        *reinterpret_cast<u32x4*>(U + static_cast<size_t>(m) * N + n) = v;
      } else {
        for (int j = 0; j < N - n; ++j)
          U[static_cast<size_t>(m) * N + n + j] = static_cast<uint16_t>(v[j >> 1] >> (16 * (j & 1)));
      }
    }
  }
  if (part && tid < kBM) {
    const int m = m0 + tid;
    if (m < M) part[static_cast<size_t>(tn) * part_ld + m] = red[tid] + red[kBM + tid];
  }
}

// ---------------------------------------------------------------------------
// fp32 path (small workloads): 64x64 tile, 4x4 outputs per thread, VALU FMA.
// ---------------------------------------------------------------------------
constexpr int kF32Tile = 64;
constexpr int kF32K = 16;

__global__ __launch_bounds__(256)
void wo_gemm_f32_kernel(const float* __restrict__ A, const float* __restrict__ W, float* __restrict__ U,
                        float* __restrict__ part, const int32_t* __restrict__ m_dev, int M_max, int N, int K,
                        int part_ld) {
  __shared__ float As[kF32K][kF32Tile + 1];
  __shared__ float Ws[kF32K][kF32Tile + 1];
  __shared__ float red[16][kF32Tile];
  int M = m_dev ? *m_dev : M_max;
  if (M > M_max) M = M_max;
  const int m0 = blockIdx.y * kF32Tile;
  const int n0 = blockIdx.x * kF32Tile;
  if (m0 >= M) return;
  const int tx = threadIdx.x & 15;  // n group
  const int ty = threadIdx.x >> 4;  // m group
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += kF32K) {
    for (int e = threadIdx.x; e < kF32Tile * kF32K; e += 256) {
      const int r = e / kF32K, kk = e % kF32K;
      const int m = m0 + r, n = n0 + r, k = k0 + kk;
      As[kk][r] = (m < M && k < K) ? A[static_cast<size_t>(m) * K + k] : 0.f;
      Ws[kk][r] = (n < N && k < K) ? W[static_cast<size_t>(n) * K + k] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kF32K; ++kk) {
      float a[4], w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) { a[i] = As[kk][ty * 4 + i]; w[i] = Ws[kk][tx * 4 + i]; }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], w[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty * 4 + i;
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx * 4 + j;
      if (n < N) {
        ss += acc[i][j] * acc[i][j];
        if (m < M) U[static_cast<size_t>(m) * N + n] = acc[i][j];
      }
    }
    red[tx][ty * 4 + i] = ss;
  }
  __syncthreads();
  if (part && threadIdx.x < kF32Tile) {
    const int m = m0 + threadIdx.x;
    float s = 0.f;
    for (int j = 0; j < 16; ++j) s += red[j][threadIdx.x];
    if (m < M) part[static_cast<size_t>(blockIdx.x) * part_ld + m] = s;
  }
}

__global__ __launch_bounds__(64)
void score_finalize_kernel(const float* __restrict__ part, int n_parts, int part_ld,
                           const int32_t* __restrict__ m_dev, int M_max, float* __restrict__ score) {
  int M = m_dev ? *m_dev : M_max;
  if (M > M_max) M = M_max;
  const int m = blockIdx.x * 64 + threadIdx.x;
  if (m >= M) return;
  // Partials are added in tile order; the loads of a group of 8 are issued together.
  float s = 0.f;
  int t = 0;
  for (; t + 8 <= n_parts; t += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = part[static_cast<size_t>(t + u) * part_ld + m];
#pragma unroll
    for (int u = 0; u < 8; ++u) s += v[u];
  }
  for (; t < n_parts; ++t) s += part[static_cast<size_t>(t) * part_ld + m];
  score[m] = sqrtf(s);
}

}  // namespace

namespace {

// Compute units of the current device, queried once per device.
int device_cus() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cache[kMaxDevices];  // 0 = not queried yet
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

// Column tile for the bf16 path: the width whose whole waves of workgroups
// (one per CU) cost least, a wave of 224-wide tiles counting 224/256 of a
// wave of 256-wide ones times 1.06 (the 224-wide kernel's lower MFMA
// efficiency, measured).  (With 256 CUs: 8192 x 3584 takes 224-wide tiles,
// 4096 x 4096, 39321 x 3584 and 131072 x 3584 take 256-wide ones.)
int bf16_tile_n(int M, int N) {
  const long tm = (M + kBM - 1) / kBM;
  const long cus = device_cus();
  const long w256 = (tm * ((N + kBN - 1) / kBN) + cus - 1) / cus;
  const long w224 = (tm * ((N + kBN224 - 1) / kBN224) + cus - 1) / cus;
  return w224 * kBN224 * 106 < w256 * kBN * 100 ? kBN224 : kBN;
}

}  // namespace

int wo_gemm_parts(int dtype, int N) {
  // Upper bound over the column tiles the launcher may pick (sizes the workspace).
  if (dtype == 1) return (N + kBN224 - 1) / kBN224;
  return (N + kF32Tile - 1) / kF32Tile;
}

hipError_t launch_wo_gemm(int dtype, const void* A, const void* W, void* U, float* score, float* part,
                          const int32_t* m_dev, int M_max, int N, int K, hipStream_t stream) {
  if (M_max <= 0) return hipSuccess;
  int parts;
  if (dtype == 1) {
    const int bn = bf16_tile_n(M_max, N);
    parts = (N + bn - 1) / bn;
    const int tm = (M_max + kBM - 1) / kBM;
    if (bn == kBN224)
      hipLaunchKernelGGL(wo_gemm_bf16_n224_kernel, dim3(tm * parts), dim3(kGemmThreads), 0, stream,
                         static_cast<const uint16_t*>(A), static_cast<const uint16_t*>(W),
                         static_cast<uint16_t*>(U), score ? part : nullptr, m_dev, M_max, N, K, parts, M_max);
    else
      hipLaunchKernelGGL(wo_gemm_bf16_kernel, dim3(tm * parts), dim3(kGemmThreads), 0, stream,
                         static_cast<const uint16_t*>(A), static_cast<const uint16_t*>(W),
                         static_cast<uint16_t*>(U), score ? part : nullptr, m_dev, M_max, N, K, parts, M_max);
  } else {
    parts = (N + kF32Tile - 1) / kF32Tile;
    hipLaunchKernelGGL(wo_gemm_f32_kernel, dim3(parts, (M_max + kF32Tile - 1) / kF32Tile), dim3(256), 0, stream,
                       static_cast<const float*>(A), static_cast<const float*>(W), static_cast<float*>(U),
                       score ? part : nullptr, m_dev, M_max, N, K, M_max);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !score) return e;
  hipLaunchKernelGGL(score_finalize_kernel, dim3((M_max + 63) / 64), dim3(64), 0, stream, part, parts, M_max,
                     m_dev, M_max, score);
  return hipGetLastError();
}

}  // namespace dash
