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
// bf16 kernel: 256 threads = 4 waves, 128 queries of one q-head per workgroup
// (32 per wave), 64 keys per step.  Scores are computed transposed,
// S^T = K · Q^T on v_mfma_f32_32x32x16_bf16, so each lane owns one query and
// 32 of the step's keys: the softmax max and sum stay in registers, and the
// partner half-wave's maximum is fetched only on the rare steps where the lazy
// reference maximum has to move.  The query is pre-scaled into exp2
// units and the score accumulators start at -m, so P is a bare exp2.  The
// output is accumulated transposed too, O^T += V^T · P^T, where P^T is fed
// straight from the score accumulators (rounded to bf16) as the B operand and
// V^T comes from transposing LDS reads (ds_read_b64_tr_b16) of the V tile.
// K and V tiles go from global memory straight into LDS (buffer loads to LDS,
// no register staging; rows past the key count read as zeros through the
// buffer range) into a ring of two K and two V tiles, K two steps ahead and V
// one; rows are XOR-swizzled so the operand reads are free of bank conflicts,
// and one barrier separates steps.  Workgroups are ordered heaviest-first
// (causal work grows with the query position) and the q-heads that share a
// kv-head are placed on the same XCD so they share its L2.
#include "dash_common.h"
#include "dash_kernels.h"

namespace dash {

namespace {

constexpr int kAttnThreads = 256;
constexpr int kBQ = 128;  // queries per workgroup
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
  static constexpr int kLoadsPerWave = kTileBytes / 1024 / (kAttnThreads / 64);
  static constexpr int kRowsPerKiB = 1024 / kRowBytes;
  static constexpr int kTotal = 4 * kTileBytes;         // K[2] + V[2]
  static constexpr int kORow = D + 8;                   // output staging row (bf16 elements)
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

// Direct global->LDS loads of one K or V tile: each wave moves kLoadsPerWave
// KiB; lane l of a 1 KiB load lands at byte 16*l, i.e. row l / kChunks, slot
// l % kChunks, and fetches the chunk the swizzle puts there.
template <int D, bool IsV>
struct TileLoader {
  using C = AttnCfg<D>;
  uint32_t voff[C::kLoadsPerWave];
  __device__ __forceinline__ void init(int kv_ld) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < C::kLoadsPerWave; ++i) {
      const int q = wave + (kAttnThreads / 64) * i;
      const int row = q * C::kRowsPerKiB + lane / C::kChunks;
      const int slot = lane % C::kChunks;
      const int chunk = IsV ? v_slot<D>(row, slot) : k_slot<D>(row, slot);
      voff[i] = static_cast<uint32_t>(row * kv_ld * 2 + chunk * 16);
    }
  }
  __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t src, unsigned char* tile, uint32_t tile_off) const {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
    for (int i = 0; i < C::kLoadsPerWave; ++i) {
      const int q = wave + (kAttnThreads / 64) * i;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(src, (__attribute__((address_space(3))) void*)(tile + q * 1024), 16,
                                               voff[i], tile_off, 0, 0);
    }
  }
};

typedef short i16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ i16x4 lds_read_tr16(const unsigned char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p));
}

template <int D>
__global__ __launch_bounds__(kAttnThreads, 2)
void attn_fwd_bf16_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                          const uint16_t* __restrict__ V, uint16_t* __restrict__ O,
                          const int32_t* __restrict__ q_pos, const int32_t* __restrict__ n_dev, int n_q_max,
                          int n_kv, int Hq, int Hkv, float c_log2, AttnBatch bt) {
  using C = AttnCfg<D>;
  __shared__ __attribute__((aligned(1024))) unsigned char lds[C::kTotal];

  const int64_t b = blockIdx.y;
  const int q_ld = Hq * D;
  const int kv_ld = Hkv * D;
  int n_q, pos_base;
  bt.locate(b, n_dev, n_q_max, n_kv, q_ld, kv_ld, Q, O, q_pos, K, V, n_q, pos_base);
  const int n_qt = (n_q_max + kBQ - 1) / kBQ;
  const int g = Hq / Hkv;
  int qt, h;
  attn_tile_of(blockIdx.x, n_qt, Hkv, g, qt, h);
  const int q0 = qt * kBQ;
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

  const int qrow = q0 + wave * 32 + l32;
  const int qrow_c = min(qrow, n_q - 1);
  const int q_src = bt.q_rows ? min(max(bt.q_rows[b * bt.qp_bs + qrow_c], 0), bt.q_rows_n - 1) : qrow_c;
  const int my_pos = q_pos ? q_pos[qrow_c] - pos_base : qrow_c;
  const int w_first = min(q0 + wave * 32, n_q - 1);
  const int w_last = min(q0 + wave * 32 + 31, n_q - 1);
  const int wave_pmin = q_pos ? q_pos[w_first] - pos_base : w_first;
  const int wave_pmax = q_pos ? q_pos[w_last] - pos_base : w_last;
  const int b_last = min(q0 + kBQ - 1, n_q - 1);
  const int block_pmax = q_pos ? q_pos[b_last] - pos_base : b_last;
  const int kv_end = min(n_kv, block_pmax + 1);
  const int n_tiles = (kv_end + kBKV - 1) / kBKV;
  // Tiles this wave computes (keys k0 <= wave_pmax) and the first one that
  // holds a key past some query of the wave (needs the causal mask).
  const int n_w = min(n_tiles, wave_pmax / kBKV + 1);
  const int j_mask = min(n_w, (wave_pmin + 1) / kBKV);

  unsigned char* kbuf0 = lds;
  unsigned char* vbuf0 = lds + 2 * C::kTileBytes;
  auto kbuf = [&](int i) { return kbuf0 + (i & 1) * C::kTileBytes; };
  auto vbuf = [&](int i) { return vbuf0 + (i & 1) * C::kTileBytes; };
  TileLoader<D, false> kload;
  TileLoader<D, true> vload;
  kload.init(kv_ld);
  vload.init(kv_ld);
  const uint32_t tile_bytes = static_cast<uint32_t>(kBKV) * row_bytes;

  // Prologue loads: K(0), K(1), V(0).
  kload.issue(k_src, kbuf(0), 0u);
  if (n_tiles > 1) kload.issue(k_src, kbuf(1), tile_bytes);
  vload.issue(v_src, vbuf(0), 0u);

  // This lane's query as the B operand of S^T = K Q^T: 8 dims per k-step,
  // pre-multiplied by log2(e)/sqrt(D) (rounded to bf16) so the scores come out
  // in exp2 units.
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

  // K operand offsets: row kb*32 + l32, chunk 2*ks + hi (the kb term is an immediate).
  int koff[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) koff[ks] = l32 * C::kRowBytes + 16 * k_slot<D>(l32, 2 * ks + hi);
  // V^T operand (transposing reads): 16-lane group grp = (l32 / 16) covers d = db*32 + 16*grp .. +15;
  // source lane j = lane % 16 reads key row kb0 + j/4, d chunk db*32 + 16*grp + 4*(j%4).
  const int tj = lane & 15;
  const int tgrp = (lane >> 4) & 1;
  int voffs[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    const int row = (tj >> 2) + 4 * hi;  // row within the tile for key step 0, part 0
    const int e = db * 32 + 16 * tgrp + 4 * (tj & 3);  // first d element read
    voffs[db] = row * C::kRowBytes + 16 * v_slot<D>(row, e >> 3) + 2 * (e & 7);
  }

  // S^T - m for one key tile: 2 blocks of 32 keys x this wave's 32 queries; the
  // first MFMA of each block takes its accumulator from m_neg (-m, m = this
  // lane's reference maximum, kept in a register block so no per-step fill is
  // needed), so the softmax numerator is a bare exp2.
  auto qk = [&](const unsigned char* kst, f32x16 (&s)[2], const f32x16& init) {
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(kst + koff[ks] + kb * 32 * C::kRowBytes);
        s[kb] = mfma32x32x16(a, qreg[ks], ks == 0 ? init : s[kb]);
      }
  };

  // Causal mask of a tile: keys past this lane's query position get -inf.
  auto mask = [&](f32x16 (&s)[2], int k0) {
    const int lim = my_pos - k0 - hi * 4;  // key offset c is visible iff c <= lim
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int c = kb * 32 + (r >> 2) * 8 + (r & 3);
        s[kb][r] = c > lim ? -__builtin_inff() : s[kb][r];
      }
  };

  // Maximum of a (masked) score tile; moves the lazy reference maximum when the
  // tile exceeds it by more than 2^kLazyLog2 in exp2 units (P then stays below
  // 2^kLazyLog2) and rescales the accumulators for it.  Called on tile j+1 at
  // the end of step j, so step j+1 itself needs no branch.
  // The tile holds S - m_run; `first` marks the first tile (m_run not set yet).
  auto update_max = [&](f32x16 (&s)[2], bool first) {
    float mx = s[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    // The two half-waves hold the same queries' other keys.  Only when some
    // lane's own half exceeds the slack (or on the first tile) is the full
    // row maximum needed, so the exchange sits inside the rare branch.
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
  };

  // Softmax numerator of a tile in place: P = exp2(S - m_run).
  auto softmax = [&](f32x16 (&s)[2]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = __builtin_amdgcn_exp2f(s[kb][r]);
  };

  // O^T += V^T P^T for one tile: P rounded to bf16 as the B operand; the V^T
  // operand (8 keys of one d per lane) comes from two transposing reads.  The
  // softmax denominator adds the same rounded P (two at a time with a bf16 dot).
  auto pv = [&](const f32x16 (&s)[2], const unsigned char* vst) {
    const bf16x2 ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
    float psum = 0.f;
#pragma unroll
    for (int stp = 0; stp < 4; ++stp) {
      const int kb = stp >> 1;
      const int sub = stp & 1;
      u32x4 pw;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        bf16x2 pr;
        pr[0] = static_cast<__bf16>(s[kb][8 * sub + 2 * t]);
        pr[1] = static_cast<__bf16>(s[kb][8 * sub + 2 * t + 1]);
        psum = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, psum, false);
        pw[t] = __builtin_bit_cast(uint32_t, pr);
      }
      const bf16x8 pb = __builtin_bit_cast(bf16x8, pw);
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        // keys 16*stp + 4*hi + (0..3) and 16*stp + 8 + 4*hi + (0..3)
        const i16x4 lo = lds_read_tr16(vst + voffs[db] + (16 * stp) * C::kRowBytes);
        const i16x4 up = lds_read_tr16(vst + voffs[db] + (16 * stp + 8) * C::kRowBytes);
        const u32x4 av = {__builtin_bit_cast(u32x2, lo)[0], __builtin_bit_cast(u32x2, lo)[1],
                          __builtin_bit_cast(u32x2, up)[0], __builtin_bit_cast(u32x2, up)[1]};
        o[db] = mfma32x32x16(__builtin_bit_cast(bf16x8, av), pb, o[db]);
      }
    }
    l_run += psum;
  };

  // Step j: wait for K(j+1) and V(j), refill the freed buffers with K(j+2) and
  // V(j+1); then, in one basic block, the scores of tile j+1 (MFMA) run beside
  // the softmax of tile j (vector ALU) and O += P V for tile j follows while the
  // maximum of tile j+1 is taken.  Tile j+1's reference maximum (and any
  // accumulator rescale) is settled at the end of the step.
  auto step = [&](int j, f32x16 (&s_cur)[2], f32x16 (&s_nxt)[2]) {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's loads of K(j+1), V(j)
    __builtin_amdgcn_s_barrier();        // everyone's; and everyone is past step j-1
    if (j + 2 < n_tiles) kload.issue(k_src, kbuf(j), static_cast<uint32_t>(j + 2) * tile_bytes);
    if (j + 1 < n_tiles) vload.issue(v_src, vbuf(j + 1), static_cast<uint32_t>(j + 1) * tile_bytes);
    // The score MFMAs (which wait on their K operand reads) run at raised wave
    // priority, so the SIMD's other wave fills in with its softmax and P V work
    // rather than competing for the same issue slots.
    if (j + 1 < j_mask) {  // steady state: tile j+1 fully visible
      __builtin_amdgcn_s_setprio(1);
      qk(kbuf(j + 1), s_nxt, m_neg);
      __builtin_amdgcn_s_setprio(0);
      softmax(s_cur);
      pv(s_cur, vbuf(j));
      update_max(s_nxt, false);
    } else {
      if (j + 1 < n_w) {
        __builtin_amdgcn_s_setprio(1);
        qk(kbuf(j + 1), s_nxt, m_neg);
        __builtin_amdgcn_s_setprio(0);
      }
      if (j < n_w) {
        softmax(s_cur);
        pv(s_cur, vbuf(j));
      }
      if (j + 1 < n_w) {
        if (j + 1 >= j_mask) mask(s_nxt, (j + 1) * kBKV);
        update_max(s_nxt, false);
      }
    }
  };

  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): query registers and prologue tiles
  __builtin_amdgcn_s_barrier();
  f32x16 sa[2], sb[2];
  if (n_w > 0) {
    qk(kbuf(0), sa, m_neg);
    if (j_mask == 0) mask(sa, 0);
    update_max(sa, true);
  }
  int j = 0;
  for (; j + 1 < n_tiles; j += 2) {
    step(j, sa, sb);
    step(j + 1, sb, sa);
  }
  if (j < n_tiles) step(j, sa, sb);

  // Normalise and stage the 128 x D output tile through LDS for 16-byte stores.
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = 1.f / l_tot;
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __syncthreads();                     // every wave is done with the K/V buffers
  uint16_t* ot = reinterpret_cast<uint16_t*>(lds);
  const int ql = wave * 32 + l32;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const int d = db * 32 + gq * 8 + hi * 4;
      u32x2 pk;
      pk[0] = pack_bf16x2(o[db][gq * 4 + 0] * inv, o[db][gq * 4 + 1] * inv);
      pk[1] = pack_bf16x2(o[db][gq * 4 + 2] * inv, o[db][gq * 4 + 3] * inv);
      *reinterpret_cast<u32x2*>(ot + ql * C::kORow + d) = pk;
    }
  __syncthreads();
  constexpr int kOutChunks = kBQ * D / 8;
#pragma unroll
  for (int i = 0; i < kOutChunks / kAttnThreads; ++i) {
    const int c = tid + i * kAttnThreads;
    const int row = c / (D / 8);
    const int dc = c % (D / 8);
    const int q = q0 + row;
    if (q < n_q)
      *reinterpret_cast<u32x4*>(O + static_cast<size_t>(q) * q_ld + h * D + dc * 8) =
          *reinterpret_cast<const u32x4*>(ot + row * C::kORow + dc * 8);
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
    const int n_qt = (n_q_max + kBQ - 1) / kBQ;
    const dim3 grid(n_qt * Hq, B);
    const float c = scale * 1.4426950408889634f;
    auto q = static_cast<const uint16_t*>(Q);
    auto k = static_cast<const uint16_t*>(K);
    auto v = static_cast<const uint16_t*>(V);
    auto o = static_cast<uint16_t*>(O);
    if (D == 128)
      hipLaunchKernelGGL(attn_fwd_bf16_kernel<128>, grid, dim3(kAttnThreads), 0, stream, q, k, v, o, q_pos, n_dev,
                         n_q_max, n_kv, Hq, Hkv, c, bt);
    else if (D == 64)
      hipLaunchKernelGGL(attn_fwd_bf16_kernel<64>, grid, dim3(kAttnThreads), 0, stream, q, k, v, o, q_pos, n_dev,
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
