// Causal grouped-query attention for the DASH prefill path (gfx950).
//
// Full-length layers and post-halt layers share one kernel.  Queries carry
// their original token positions (identity for a full-length layer); key row r
// sits at position r of the K/V it is given.  Key r is visible to a query at
// position p iff r <= p.  This covers:
//   * the full-length layer: queries 0..S-1, keys 0..S-1;
//   * post-halt with the pruned KV cache (keys and values compacted at the same
//     ascending positions as the queries): causal in compacted order, which is
//     the same order because the active set is ascending — CSDN explainer
//     "DASH：基于注意力增量的Transformer令牌压缩，实现长序列推理高效加速", §3.1
//     step 4 and §5.1 (only active tokens are computed and cached);
//   * post-halt with the full KV cache (halted tokens keep their K/V but are no
//     longer queries) — forum summary "DASH：通过注意力动态监测实现长上下文高效预填充",
//     section 选择性停止机制.
//
// bf16 kernel: 512 threads = 8 waves, 256 queries of one q-head per workgroup
// (32 per wave), 64 keys per step, one workgroup per CU.  Scores are computed
// transposed, S^T = K · Q^T on v_mfma_f32_32x32x16_bf16, so each lane owns one
// query and 32 of the step's keys: the softmax max and sum stay in registers,
// and the partner half-wave's maximum is fetched only on the rare steps where
// the lazy reference maximum has to move.  The query is pre-scaled into exp2
// units and the score accumulators start at -m, so P is a bare exp2.  The
// output is accumulated transposed too, O^T += V^T · P^T, with P^T (rounded to
// bf16) as the B operand and V^T from transposing LDS reads
// (ds_read_b64_tr_b16).  The eight waves form two groups that alternate, one
// phase apart, between matrix phases (the scores of the next tile and P V of
// the current one) and softmax phases, so the two waves sharing a SIMD keep
// its matrix pipe fed in turn (details at the kernel).  K and V tiles go from
// global memory straight into LDS (buffer loads to LDS, no register staging;
// rows past the key count read as zeros through the buffer range); rows are
// XOR-swizzled so the operand reads are free of bank conflicts.  Workgroups
// are ordered heaviest-first (causal work grows with the query position) and
// the q-heads that share a kv-head are placed on the same XCD so they share
// its L2.
#include <type_traits>

#include "dash_common.h"
#include "dash_kernels.h"

namespace dash {

namespace {

constexpr int kBKV = 64;  // keys per step
constexpr float kLazyLog2 = 8.0f;  // slack of the lazily updated softmax maximum

// Logical (query tile, q-head) of workgroup `bid`: pairs (query tile, kv-head)
// are enumerated heaviest query tile first; the g q-heads of a pair land on
// workgroup ids that are equal mod 8 (one XCD).
__device__ __forceinline__ void attn_tile_of(int bid, int n_qt, int Hkv, int g, int& qt, int& h) {
  const int pairs = n_qt * Hkv;
  const int full = pairs / 8;
  const int grp = 8 * g;
  int p, j;
  if (bid < full * grp) {
    const int gi = bid / grp, w = bid - gi * grp;
    j = w >> 3;
    p = gi * 8 + (w & 7);
  } else {
    const int r = pairs - full * 8;
    const int w = bid - full * grp;
    j = w / r;
    p = full * 8 + (w - j * r);
  }
  const int kvh = p % Hkv;
  qt = n_qt - 1 - p / Hkv;
  h = kvh * g + j;
}

// Buffer resource over `bytes` bytes from `base`: loads past the end return 0,
// which is how rows beyond the key count read as zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), static_cast<int>(bytes),
                                           0x00020000);
}

template <int D>
struct AttnCfg {
  static constexpr int kRowBytes = D * 2;               // K and V rows in LDS (unpadded, swizzled)
  static constexpr int kChunks = kRowBytes / 16;        // 16-byte chunks per row
  static constexpr int kRowsPerLine = 256 / kRowBytes;  // rows per 64-bank line
  static constexpr int kTileBytes = kBKV * kRowBytes;   // one K or V tile
  static constexpr int kRowsPerKiB = 1024 / kRowBytes;
};

// K rows: chunk c of row r sits at slot c ^ ((r / kRowsPerLine) % kChunks), so
// the 16 consecutive rows of one 16-byte operand read hit distinct banks.
template <int D>
__device__ __forceinline__ int k_slot(int r, int c) {
  using C = AttnCfg<D>;
  return c ^ ((r / C::kRowsPerLine) % C::kChunks);
}

// V rows: chunk c of row r sits at slot c ^ (4 * ((r / kRowsPerLine) % (kChunks / 4))),
// so the four rows x 64 bytes that 32 lanes fetch in one transposing read
// (ds_read_b64_tr_b16) hit distinct banks.
template <int D>
__device__ __forceinline__ int v_slot(int r, int c) {
  using C = AttnCfg<D>;
  return c ^ (4 * ((r / C::kRowsPerLine) % (C::kChunks / 4)));
}

typedef short i16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ i16x4 lds_read_tr16(const unsigned char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p));
}

// ---------------------------------------------------------------------------
// bf16 kernel, two wave groups in alternation.  512 threads = 8 waves, 256
// queries of one q-head per workgroup (32 per wave), one workgroup per CU, so
// each SIMD holds two waves; they are made one wave of group 0 and one of
// group 1.  Every wave runs the same sequence of phases for key tile j:
//   M(j): the scores of tile j+1 (S^T = K Q^T, 16 MFMAs) and O^T += V^T P^T
//         for tile j (16 MFMAs), at raised wave priority;
//   V(j+1): mask, lazy maximum, exp2, bf16 packing and row sum of tile j+1
//         (vector ALU only), plus this group's share of the tile loads;
// with a workgroup barrier after each phase.  Group 1 starts one phase later
// than group 0, so while one wave of a SIMD issues matrix instructions its
// partner runs the softmax of the other group; the matrix pipe sees the two
// waves' MFMA phases back to back.
// K and V tiles sit in rings of three LDS buffers each, every buffer its own
// __shared__ array and the loop unrolled by three so each buffer is fixed at
// compile time: the compiler then sees that a transposing V read does not
// touch the buffer a tile load is filling and does not wait for the load.
// Group 0 loads K tiles during its V phases (K(t+2) while publishing K(t+1));
// group 1 loads V tiles (V(t+2), publishing V(t+1)).
// ---------------------------------------------------------------------------
constexpr int kPPThreads = 512;
constexpr int kPPQ = 256;  // queries per workgroup

// A K or V tile moved by one group of four waves: the wave in group slot gw
// moves 1 KiB pieces gw, gw + 4, ...: lane l of a piece lands at byte 16*l,
// i.e. row l / kChunks, slot l % kChunks, and fetches the chunk the swizzle
// puts there.  One loader per wave, set up for the tiles its group moves.
template <int D>
struct GroupTileLoader {
  using C = AttnCfg<D>;
  static constexpr int kLoads = C::kTileBytes / 1024 / 4;
  uint32_t voff[kLoads];
  int gw;  // this wave's slot (0-3) within its group
  __device__ __forceinline__ void init(int kv_ld, bool is_v, int slot_in_group) {
    gw = slot_in_group;
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int q = gw + 4 * i;
      const int row = q * C::kRowsPerKiB + lane / C::kChunks;
      const int slot = lane % C::kChunks;
      const int chunk = is_v ? v_slot<D>(row, slot) : k_slot<D>(row, slot);
      voff[i] = static_cast<uint32_t>(row * kv_ld * 2 + chunk * 16);
    }
  }
  __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t src, unsigned char* tile, uint32_t tile_off) const {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int q = gw + 4 * i;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(src, (__attribute__((address_space(3))) void*)(tile + q * 1024), 16,
                                               voff[i], tile_off, 0, 0);
    }
  }
};

template <int N>
using Slot = std::integral_constant<int, N>;

template <int D>
__global__ __launch_bounds__(kPPThreads, 2)
void attn_fwd_bf16_pp_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                             const uint16_t* __restrict__ V, uint16_t* __restrict__ O,
                             const int32_t* __restrict__ q_pos, const int32_t* __restrict__ n_dev, int n_q_max,
                             int n_kv, int Hq, int Hkv, float c_log2, AttnBatch bt) {
  using C = AttnCfg<D>;
  // The LDS allocator places these arrays in name order: the V ring (named to
  // come first) then sits below 64 KiB, so its transposing reads carry the
  // buffer's place as an immediate offset instead of an address add.
  __shared__ __attribute__((aligned(1024))) unsigned char lds_a_v0[C::kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char lds_a_v1[C::kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char lds_a_v2[C::kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char lds_b_k0[C::kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char lds_b_k1[C::kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char lds_b_k2[C::kTileBytes];
  auto kbuf = [&](auto n) -> unsigned char* {
    if constexpr (decltype(n)::value == 0) return lds_b_k0;
    else if constexpr (decltype(n)::value == 1) return lds_b_k1;
    else return lds_b_k2;
  };
  auto vbuf = [&](auto n) -> unsigned char* {
    if constexpr (decltype(n)::value == 0) return lds_a_v0;
    else if constexpr (decltype(n)::value == 1) return lds_a_v1;
    else return lds_a_v2;
  };

  const int64_t b = blockIdx.y;
  const int q_ld = Hq * D;
  const int kv_ld = Hkv * D;
  int n_q, pos_base;
  bt.locate(b, n_dev, n_q_max, n_kv, q_ld, kv_ld, Q, O, q_pos, K, V, n_q, pos_base);
  const int n_qt = (n_q_max + kPPQ - 1) / kPPQ;
  const int g = Hq / Hkv;
  int qt, h;
  attn_tile_of(blockIdx.x, n_qt, Hkv, g, qt, h);
  const int q0 = qt * kPPQ;
  if (q0 >= n_q) return;
  const int kvh = h / g;
  K += static_cast<int64_t>(kvh) * D;
  V += static_cast<int64_t>(kvh) * D;
  const uint32_t row_bytes = static_cast<uint32_t>(kv_ld) * 2u;
  // bytes from this kv-head's first element to the end of the last key row;
  // loads past it (rows beyond the key count) return zeros
  const uint32_t kv_bytes = n_kv > 0 ? static_cast<uint32_t>(n_kv - 1) * row_bytes + D * 2u : 0u;
  const __amdgpu_buffer_rsrc_t k_src = make_rsrc(K, kv_bytes);
  const __amdgpu_buffer_rsrc_t v_src = make_rsrc(V, kv_bytes);

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  // Groups by SIMD: the two waves the hardware placed on each SIMD become one
  // wave of group 0 and one of group 1 (lower wave index first), and the SIMD
  // index is the wave's slot within its group.  The SIMD of a wave is read from
  // the HW_ID register (bits 5:4).  Should the waves not pair up two per SIMD,
  // the split falls back to waves 0-3 / 4-7.
  __shared__ int simd_of[kPPThreads / 64];
  const int my_simd = static_cast<int>((__builtin_amdgcn_s_getreg((4) | (4 << 6) | ((2 - 1) << 11))) & 3u);
  if (lane == 0) simd_of[wave] = my_simd;
  __syncthreads();
  int grp = wave >> 2, gslot = wave & 3;
  {
    bool paired = true;
    int rank = 0;
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) {
      int cnt = 0;
#pragma unroll
      for (int w2 = 0; w2 < kPPThreads / 64; ++w2) cnt += simd_of[w2] == s2;
      paired = paired && cnt == 2;
    }
#pragma unroll
    for (int w2 = 0; w2 < kPPThreads / 64; ++w2) rank += (w2 < wave && simd_of[w2] == my_simd);
    if (paired) {
      grp = rank;
      gslot = my_simd;
    }
  }
  grp = __builtin_amdgcn_readfirstlane(grp);
  gslot = __builtin_amdgcn_readfirstlane(gslot);

  const int qrow = q0 + wave * 32 + l32;
  const int qrow_c = min(qrow, n_q - 1);
  const int q_src = bt.q_rows ? min(max(bt.q_rows[b * bt.qp_bs + qrow_c], 0), bt.q_rows_n - 1) : qrow_c;
  const int my_pos = q_pos ? q_pos[qrow_c] - pos_base : qrow_c;
  const int w_first = min(q0 + wave * 32, n_q - 1);
  const int w_last = min(q0 + wave * 32 + 31, n_q - 1);
  const int wave_pmin = q_pos ? q_pos[w_first] - pos_base : w_first;
  const int wave_pmax = q_pos ? q_pos[w_last] - pos_base : w_last;
  const int b_last = min(q0 + kPPQ - 1, n_q - 1);
  const int block_pmax = q_pos ? q_pos[b_last] - pos_base : b_last;
  const int kv_end = min(n_kv, block_pmax + 1);
  const int n_tiles = (kv_end + kBKV - 1) / kBKV;
  if (n_tiles <= 0) return;
  // Tiles this wave computes (keys k0 <= wave_pmax) and the first one that
  // holds a key past some query of the wave (needs the causal mask).
  const int n_w = min(n_tiles, wave_pmax / kBKV + 1);
  const int j_mask = min(n_w, (wave_pmin + 1) / kBKV);

  GroupTileLoader<D> ld;  // group 0 moves K tiles, group 1 V tiles
  constexpr int kLoads = GroupTileLoader<D>::kLoads;
  ld.init(kv_ld, grp == 1, gslot);
  const uint32_t tile_bytes = static_cast<uint32_t>(kBKV) * row_bytes;

  // Prologue loads: K(0), K(1) by group 0; V(0), V(1) by group 1.
  if (grp == 0) {
    ld.issue(k_src, lds_b_k0, 0u);
    if (n_tiles > 1) ld.issue(k_src, lds_b_k1, tile_bytes);
  } else {
    ld.issue(v_src, lds_a_v0, 0u);
    if (n_tiles > 1) ld.issue(v_src, lds_a_v1, tile_bytes);
  }

  // This lane's query as the B operand of S^T = K Q^T, pre-multiplied by
  // log2(e)/sqrt(D) (rounded to bf16) so the scores come out in exp2 units.
  bf16x8 qreg[D / 16];
  {
    const uint16_t* qp = Q + static_cast<size_t>(q_src) * q_ld + h * D + hi * 8;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const bf16x8 raw = *reinterpret_cast<const bf16x8*>(qp + ks * 16);
#pragma unroll
      for (int e = 0; e < 8; ++e) qreg[ks][e] = static_cast<__bf16>(static_cast<float>(raw[e]) * c_log2);
    }
  }

  f32x16 o[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[i][r] = 0.f;
  float m_run = 0.f;  // reference maximum (exp2 units); score tiles hold S - m_run
  f32x16 m_neg;       // -m_run in every element: the score MFMAs' initial accumulator
#pragma unroll
  for (int r = 0; r < 16; ++r) m_neg[r] = 0.f;
  float l_run = 0.f;
  u32x4 pk[4];        // P of the tile being multiplied, bf16 pairs (B operands of P V)
  u32x4 vpre[D / 32]; // V^T operands of that tile's first key step, read ahead of its M phase
  f32x16 s[2];        // scores of the tile after it (S^T - m, then in place through the softmax)

  int koff[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) koff[ks] = l32 * C::kRowBytes + 16 * k_slot<D>(l32, 2 * ks + hi);
  const int tj = lane & 15;
  const int tgrp = (lane >> 4) & 1;
  int voffs[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    const int row = (tj >> 2) + 4 * hi;
    const int e = db * 32 + 16 * tgrp + 4 * (tj & 3);
    voffs[db] = row * C::kRowBytes + 16 * v_slot<D>(row, e >> 3) + 2 * (e & 7);
  }

  auto qk = [&](const unsigned char* kst, f32x16 (&s)[2]) {
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(kst + koff[ks] + kb * 32 * C::kRowBytes);
        s[kb] = mfma32x32x16(a, qreg[ks], ks == 0 ? m_neg : s[kb]);
      }
  };

  auto pv = [&](const unsigned char* vst) {
#pragma unroll
    for (int stp = 0; stp < 4; ++stp) {
      const bf16x8 pb = __builtin_bit_cast(bf16x8, pk[stp]);
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        u32x4 av;
        if (stp == 0) {
          av = vpre[db];
        } else {
          const i16x4 lo = lds_read_tr16(vst + voffs[db] + (16 * stp) * C::kRowBytes);
          const i16x4 up = lds_read_tr16(vst + voffs[db] + (16 * stp + 8) * C::kRowBytes);
          av = u32x4{__builtin_bit_cast(u32x2, lo)[0], __builtin_bit_cast(u32x2, lo)[1],
                     __builtin_bit_cast(u32x2, up)[0], __builtin_bit_cast(u32x2, up)[1]};
        }
        o[db] = mfma32x32x16(__builtin_bit_cast(bf16x8, av), pb, o[db]);
      }
    }
  };
  // The V^T operands of the first key step of the tile in V buffer vst, read
  // at the end of the softmax phase (the tile was published a phase earlier),
  // so the next M phase starts on operands already in registers.
  auto prefetch_v = [&](const unsigned char* vst) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const i16x4 lo = lds_read_tr16(vst + voffs[db]);
      const i16x4 up = lds_read_tr16(vst + voffs[db] + 8 * C::kRowBytes);
      vpre[db] = u32x4{__builtin_bit_cast(u32x2, lo)[0], __builtin_bit_cast(u32x2, lo)[1],
                       __builtin_bit_cast(u32x2, up)[0], __builtin_bit_cast(u32x2, up)[1]};
    }
  };

  // M phase with both products: the scores of the next tile (s) and O += P V
  // of the current one, their MFMAs interleaved; the LDS operand reads are
  // kept several MFMAs ahead (scheduling groups), since the SIMD's other wave
  // is in its vector-ALU phase and cannot cover their latency.  The P V
  // MFMAs of the first key step come first: their V operands were read in
  // the softmax phase, so they run while the first K reads are in flight.
  auto mphase = [&](const unsigned char* kst, const unsigned char* vst) {
    // 2 * (D / 16) score MFMAs (two key blocks per k-step) and 4 * (D / 32)
    // P V MFMAs (four key steps per output block): equal counts for every D
    constexpr int kN = 2 * (D / 16);
    static_assert(kN == 4 * (D / 32), "paired MFMA counts");
    auto pv_mfma = [&](int j) {  // stp = j / (D / 32), db = j % (D / 32)
      const int stp = j / (D / 32), db = j % (D / 32);
      u32x4 av;
      if (stp == 0) {
        av = vpre[db];
      } else {
        const i16x4 lo = lds_read_tr16(vst + voffs[db] + (16 * stp) * C::kRowBytes);
        const i16x4 up = lds_read_tr16(vst + voffs[db] + (16 * stp + 8) * C::kRowBytes);
        av = u32x4{__builtin_bit_cast(u32x2, lo)[0], __builtin_bit_cast(u32x2, lo)[1],
                   __builtin_bit_cast(u32x2, up)[0], __builtin_bit_cast(u32x2, up)[1]};
      }
      o[db] = mfma32x32x16(__builtin_bit_cast(bf16x8, av), __builtin_bit_cast(bf16x8, pk[stp]), o[db]);
    };
#pragma unroll
    for (int j = 0; j < D / 32; ++j) pv_mfma(j);
#pragma unroll
    for (int i = 0; i < kN; ++i) {
      const int ks = i >> 1, kb = i & 1;
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(kst + koff[ks] + kb * 32 * C::kRowBytes);
      s[kb] = mfma32x32x16(a, qreg[ks], ks == 0 ? m_neg : s[kb]);
      if (i + D / 32 < kN) pv_mfma(i + D / 32);
    }
    // 3 LDS reads per pair of MFMAs: ten reads ahead, then MFMA, two
    // reads, MFMA, one read, ...
    __builtin_amdgcn_sched_group_barrier(0x100, 10, 0);
#pragma unroll
    for (int i = 0; i < 2 * (D / 16); ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
  };

  // Softmax phase of tile t held in s: causal mask where needed, the lazily
  // updated reference maximum (rescaling O and the row sum when it moves),
  // P = exp2(S - m), rounded to bf16 into pk, and the row sum of the rounded P.
  auto vphase = [&](f32x16 (&s)[2], int t, bool first) {
    if (t >= j_mask) {
      const int lim = my_pos - t * kBKV - hi * 4;  // key offset c is visible iff c <= lim
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int c = kb * 32 + (r >> 2) * 8 + (r & 3);
          s[kb][r] = c > lim ? -__builtin_inff() : s[kb][r];
        }
    }
    float mx = s[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    if (__any(first || mx > kLazyLog2)) {
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const bool grow = first || mx > kLazyLog2;
      const float delta = grow ? mx : 0.f;
      const float alpha = first ? 0.f : __builtin_amdgcn_exp2f(-delta);
      m_run = first ? mx : m_run + delta;
#pragma unroll
      for (int r = 0; r < 16; ++r) m_neg[r] = -m_run;
      l_run *= alpha;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] -= delta;
#pragma unroll
      for (int i = 0; i < D / 32; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[i][r] *= alpha;
    }
    // row sum of P in fp32, four independent chains (a bf16 dot product here
    // would share the matrix unit's issue with the partner wave's MFMAs)
    float ps[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int stp = 0; stp < 4; ++stp) {
      const int kb = stp >> 1;
      const int sub = stp & 1;
#pragma unroll
      for (int t2 = 0; t2 < 4; ++t2) {
        const float p0 = __builtin_amdgcn_exp2f(s[kb][8 * sub + 2 * t2]);
        const float p1 = __builtin_amdgcn_exp2f(s[kb][8 * sub + 2 * t2 + 1]);
        ps[t2] += p0 + p1;
        pk[stp][t2] = pack_bf16x2(p0, p1);
      }
    }
    l_run += (ps[0] + ps[1]) + (ps[2] + ps[3]);
  };

  // This group's share of the tile loads in its V phase of tile t: group 0
  // issues K(t+2) and waits for K(t+1); group 1 the same for V.  The buffer
  // that receives tile t+2 is slot (t+2) % 3.
  auto loads = [&](auto slot2, int t) {
    if (t + 2 < n_tiles) {
      if (grp == 0) ld.issue(k_src, kbuf(slot2), static_cast<uint32_t>(t + 2) * tile_bytes);
      else ld.issue(v_src, vbuf(slot2), static_cast<uint32_t>(t + 2) * tile_bytes);
      __builtin_amdgcn_s_waitcnt(0x0F70 | kLoads);  // vmcnt(kLoads): tile t+1 is in
    } else {
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    }
  };

  auto barrier = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };

  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): query registers and prologue tiles
  barrier();
  if (n_w > 0) qk(lds_b_k0, s);
  if (grp == 0) {
    if (n_w > 0) vphase(s, 0, true);
    loads(Slot<2>{}, 0);
    prefetch_v(lds_a_v0);
  }
  barrier();
  if (grp == 1) {
    if (n_w > 0) vphase(s, 0, true);
    loads(Slot<2>{}, 0);
    prefetch_v(lds_a_v0);
    barrier();
  }

  // Step j: M(j) with K slot (j+1) % 3 and V slot j % 3, then V(j+1), whose
  // loads fill slot (j+3) % 3 = j % 3.
  auto step = [&](auto sj, int j) {
    constexpr int a = decltype(sj)::value;
    __builtin_amdgcn_s_setprio(1);
    if (j + 1 < n_w) mphase(kbuf(Slot<(a + 1) % 3>{}), vbuf(Slot<a>{}));
    else if (j < n_w) pv(vbuf(Slot<a>{}));
    __builtin_amdgcn_s_setprio(0);
    barrier();
    if (j + 1 < n_w) vphase(s, j + 1, false);
    loads(Slot<a>{}, j + 1);
    prefetch_v(vbuf(Slot<(a + 1) % 3>{}));
    barrier();
  };
  auto last = [&](auto sj, int j) {
    constexpr int a = decltype(sj)::value;
    __builtin_amdgcn_s_setprio(1);
    if (j < n_w) pv(vbuf(Slot<a>{}));
    __builtin_amdgcn_s_setprio(0);
    barrier();
  };

  int j = 0;
  for (; j + 3 <= n_tiles - 1; j += 3) {
    step(Slot<0>{}, j);
    step(Slot<1>{}, j + 1);
    step(Slot<2>{}, j + 2);
  }
  if (j < n_tiles - 1) step(Slot<0>{}, j++);
  if (j < n_tiles - 1) step(Slot<1>{}, j++);
  if (j % 3 == 0) last(Slot<0>{}, j);
  else if (j % 3 == 1) last(Slot<1>{}, j);
  else last(Slot<2>{}, j);
  if (grp == 0) barrier();  // group 1 ran one phase behind: every wave is past its last LDS read now

  // Normalise; stage each wave's 32 x D output rows through LDS (two waves per
  // buffer, 16-byte chunks XOR-swizzled by row) for 16-byte stores.
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = 1.f / l_tot;
  unsigned char* stage;
  switch (wave >> 1) {
    case 0: stage = lds_b_k0; break;
    case 1: stage = lds_b_k1; break;
    case 2: stage = lds_b_k2; break;
    default: stage = lds_a_v0; break;
  }
  stage += (wave & 1) * (32 * C::kRowBytes);
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const int c = db * 4 + gq;  // 16-byte chunk of the row
      const int cs = c ^ (l32 % C::kChunks);
      u32x2 pk2;
      pk2[0] = pack_bf16x2(o[db][gq * 4 + 0] * inv, o[db][gq * 4 + 1] * inv);
      pk2[1] = pack_bf16x2(o[db][gq * 4 + 2] * inv, o[db][gq * 4 + 3] * inv);
      *reinterpret_cast<u32x2*>(stage + l32 * C::kRowBytes + cs * 16 + hi * 8) = pk2;
    }
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's staging writes are in
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int i = 0; i < 32 * C::kChunks / 64; ++i) {
    const int cid = lane + 64 * i;
    const int row = cid / C::kChunks;
    const int c = cid % C::kChunks;
    const int q = q0 + wave * 32 + row;
    const u32x4 v = *reinterpret_cast<const u32x4*>(stage + row * C::kRowBytes + 16 * (c ^ (row % C::kChunks)));
    if (q < n_q) *reinterpret_cast<u32x4*>(O + static_cast<size_t>(q) * q_ld + h * D + c * 8) = v;
  }
}

// ---------------------------------------------------------------------------
// fp32 kernel (small workloads): one wave = 64 queries of one head; K/V tiles
// of 64 keys in LDS; each lane runs the online softmax over the keys in order.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(64)
void attn_fwd_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
                         float* __restrict__ O, const int32_t* __restrict__ q_pos,
                         const int32_t* __restrict__ n_dev, int n_q_max, int n_kv, int Hq, int Hkv, float scale,
                         AttnBatch bt) {
  __shared__ float ks[64][D];
  __shared__ float vs[64][D];
  const int64_t b = blockIdx.z;
  const int q_ld = Hq * D, kv_ld = Hkv * D;
  int n_q, pos_base;
  bt.locate(b, n_dev, n_q_max, n_kv, q_ld, kv_ld, Q, O, q_pos, K, V, n_q, pos_base);
  const int q0 = blockIdx.x * 64;
  if (q0 >= n_q) return;
  const int h = blockIdx.y;
  const int kvh = h / (Hq / Hkv);
  K += static_cast<int64_t>(kvh) * D;
  V += static_cast<int64_t>(kvh) * D;
  const int qi = q0 + threadIdx.x;
  const int qc = min(qi, n_q - 1);
  const int q_src = bt.q_rows ? min(max(bt.q_rows[b * bt.qp_bs + qc], 0), bt.q_rows_n - 1) : qc;
  const int my_pos = q_pos ? q_pos[qc] - pos_base : qc;
  const int last = min(q0 + 63, n_q - 1);
  const int pmax = q_pos ? q_pos[last] - pos_base : last;
  const int kv_end = min(n_kv, pmax + 1);
  float q[D], acc[D];
#pragma unroll
  for (int d = 0; d < D; ++d) { q[d] = Q[static_cast<size_t>(q_src) * q_ld + h * D + d] * scale; acc[d] = 0.f; }
  float m = -__builtin_inff(), l = 0.f;
  for (int k0 = 0; k0 < kv_end; k0 += 64) {
    __syncthreads();
    for (int e = threadIdx.x; e < 64 * D; e += 64) {
      const int r = e / D, d = e % D;
      const int row = k0 + r;
      ks[r][d] = row < n_kv ? K[static_cast<size_t>(row) * kv_ld + d] : 0.f;
      vs[r][d] = row < n_kv ? V[static_cast<size_t>(row) * kv_ld + d] : 0.f;
    }
    __syncthreads();
    const int kend = min(64, kv_end - k0);
    for (int r = 0; r < kend; ++r) {
      if (k0 + r > my_pos) break;
      float s = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) s = fmaf(q[d], ks[r][d], s);
      const float mn = fmaxf(m, s);
      const float a = expf(m - mn);
      const float p = expf(s - mn);
      l = l * a + p;
#pragma unroll
      for (int d = 0; d < D; ++d) acc[d] = fmaf(acc[d], a, p * vs[r][d]);
      m = mn;
    }
  }
  if (qi < n_q) {
    const float inv = 1.f / l;
#pragma unroll
    for (int d = 0; d < D; ++d) O[static_cast<size_t>(qi) * q_ld + h * D + d] = acc[d] * inv;
  }
}

}  // namespace

hipError_t launch_attention(int dtype, int B, int D, const void* Q, const void* K, const void* V, void* O,
                            const int32_t* q_pos, const int32_t* n_dev, int n_q_max, int n_kv, int Hq, int Hkv,
                            const AttnBatch& bt, hipStream_t stream) {
  if (n_q_max <= 0 || B <= 0) return hipSuccess;
  const float scale = 1.0f / sqrtf(static_cast<float>(D));
  if (dtype == 1) {
    const float c = scale * 1.4426950408889634f;
    auto q = static_cast<const uint16_t*>(Q);
    auto k = static_cast<const uint16_t*>(K);
    auto v = static_cast<const uint16_t*>(V);
    auto o = static_cast<uint16_t*>(O);
    const dim3 grid(((n_q_max + kPPQ - 1) / kPPQ) * Hq, B);
    if (D == 128)
      hipLaunchKernelGGL(attn_fwd_bf16_pp_kernel<128>, grid, dim3(kPPThreads), 0, stream, q, k, v, o, q_pos, n_dev,
                         n_q_max, n_kv, Hq, Hkv, c, bt);
    else if (D == 64)
      hipLaunchKernelGGL(attn_fwd_bf16_pp_kernel<64>, grid, dim3(kPPThreads), 0, stream, q, k, v, o, q_pos, n_dev,
                         n_q_max, n_kv, Hq, Hkv, c, bt);
    else
      return hipErrorInvalidValue;
  } else {
    const dim3 grid((n_q_max + 63) / 64, Hq, B);
    auto q = static_cast<const float*>(Q);
    auto k = static_cast<const float*>(K);
    auto v = static_cast<const float*>(V);
    auto o = static_cast<float*>(O);
    if (D == 128)
      hipLaunchKernelGGL(attn_fwd_f32_kernel<128>, grid, dim3(64), 0, stream, q, k, v, o, q_pos, n_dev, n_q_max,
                         n_kv, Hq, Hkv, scale, bt);
    else if (D == 64)
      hipLaunchKernelGGL(attn_fwd_f32_kernel<64>, grid, dim3(64), 0, stream, q, k, v, o, q_pos, n_dev, n_q_max,
                         n_kv, Hq, Hkv, scale, bt);
    else if (D == 32)
      hipLaunchKernelGGL(attn_fwd_f32_kernel<32>, grid, dim3(64), 0, stream, q, k, v, o, q_pos, n_dev, n_q_max,
                         n_kv, Hq, Hkv, scale, bt);
    else
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace dash
