// Selection kernels of the DASH prefill path (gfx950).
//
// * Top-k:  the k tokens with the largest Δattn score, written in ascending
//   position order — the single-shot halting decision of the CSDN explainer
//   "DASH：基于注意力增量的Transformer令牌压缩，实现长序列推理高效加速", §2.3 and
//   §3.1 step 3 (sort descending, keep the top K; active indices kept sorted,
//   §3.3).  Equal scores go to the lower position.
// * Order statistic: the rank-th smallest score, used as the halting
//   threshold of the selective-halting policy.
// * Threshold step: consecutive-layer counters and halting, from the forum
//   summary "DASH：通过注意力动态监测实现长上下文高效预填充", sections
//   层间更新动态监测 and 选择性停止机制.
//
// One workgroup of 1024 threads owns one row of scores (batches of at least
// 256 rows of at most 8192 aligned scores take one wave per row instead).
// Scores map to order-preserving 32-bit keys.  A radix select over LDS
// histograms finds the cut key T and how many keys equal to T must be taken:
// for rows held in registers and for a single long row, the bits shared by the
// row's smallest and largest key are settled first, then digits of up to 11
// bits follow, most significant first (long rows in a batch use 11-, 11- and
// 10-bit digits).  A final pass with a
// prefix scan of (greater-than-T, equal-to-T) counts emits the survivors in
// ascending order, so ties resolve to the lower position without any sort.
// Everything lives in one launch: no host round trip, no global atomics,
// deterministic.
#include "dash_common.h"
#include "dash_kernels.h"

namespace dash {

namespace {

constexpr int kSelThreads = 1024;  // one workgroup per row
constexpr int kWaveRowsMin = 256;  // from this many rows on, short rows take one wave each
constexpr int kSelWaves = kSelThreads / kWave;
constexpr int kBins = 2048;
// Each histogram is kept in kCopies copies, lane l counting into copy
// l % kCopies: scores cluster in a few bins, and the copies cut same-address
// LDS atomic conflicts by that factor.
constexpr int kCopies = 4;

// Order-preserving key: larger score -> larger key.  NaN -> 0 (below every
// number, including -inf whose key is 0x007fffff); -0 and +0 share one key.
// Integer-only, so the result does not depend on the denormal mode.
__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t b = __float_as_uint(f);
  const uint32_t mag = b & 0x7fffffffu;
  if (mag > 0x7f800000u) return 0u;  // NaN
  if (mag == 0u) b = 0u;             // -0 -> +0
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ float key_score(uint32_t k) {
  if (k == 0u) return __uint_as_float(0x7fc00000u);
  const uint32_t b = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(b);
}

// Inclusive scan of a 32-bit value over the 64 lanes of a wave, in registers
// (DPP): shifts by 1, 2, 4 and 8 within each row of 16 lanes, then the row
// totals are carried across rows with the row_bcast:15 / row_bcast:31 moves.
// Lanes whose DPP source does not exist read `id`, the operator's identity.
template <class Op>
__device__ __forceinline__ uint32_t wave_incl_scan_op(uint32_t v, uint32_t id, Op op) {
  const int i = static_cast<int>(id);
  v = op(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(i, static_cast<int>(v), 0x111, 0xf, 0xf, false)));
  v = op(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(i, static_cast<int>(v), 0x112, 0xf, 0xf, false)));
  v = op(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(i, static_cast<int>(v), 0x114, 0xf, 0xf, false)));
  v = op(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(i, static_cast<int>(v), 0x118, 0xf, 0xf, false)));
  v = op(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(i, static_cast<int>(v), 0x142, 0xa, 0xf, false)));
  v = op(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(i, static_cast<int>(v), 0x143, 0xc, 0xf, false)));
  return v;
}

__device__ __forceinline__ uint32_t wave_incl_scan32(uint32_t v) {
  return wave_incl_scan_op(v, 0u, [](uint32_t a, uint32_t b) { return a + b; });
}

// Inclusive wave scan of a pair of 32-bit counts packed in 64 bits (no carry
// crosses the halves: every count here is below 2^31).
__device__ __forceinline__ uint64_t wave_incl_scan(uint64_t v) {
  const uint32_t lo = wave_incl_scan32(static_cast<uint32_t>(v));
  const uint32_t hi = wave_incl_scan32(static_cast<uint32_t>(v >> 32));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// Exclusive scan of a 64-bit value over the NT threads of a workgroup; also
// returns the workgroup total.  sh_waves holds 2 * NT / 64 + 1 entries.
template <int NT>
__device__ __forceinline__ uint64_t block_excl_scan(uint64_t v, uint64_t* sh_waves, uint64_t& total) {
  constexpr int kW = NT / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = threadIdx.x / kWave;
  const uint64_t incl = wave_incl_scan(v);
  if (lane == kWave - 1) sh_waves[wid] = incl;
  __syncthreads();
  if (wid == 0) {
    uint64_t w = (lane < kW) ? sh_waves[lane] : 0ull;
    const uint64_t wi = wave_incl_scan(w);
    if (lane < kW) sh_waves[kW + lane] = wi - w;  // exclusive wave offsets
    if (lane == kW - 1) sh_waves[2 * kW] = wi;
  }
  __syncthreads();
  const uint64_t res = sh_waves[kW + wid] + incl - v;
  total = sh_waves[2 * kW];
  __syncthreads();
  return res;
}

// Find the key of the kk-th largest (1-based) among the keys visited by
// `for_keys(f)` (which calls f(key) for each of this thread's keys).  Returns
// the cut key; *take_eq = how many keys equal to it are ranked within the top
// kk (the kk - #greater lowest-position ones).
//
// Adaptive (keys held in registers, so an extra look is free): the bits every
// key shares (the common prefix of the smallest and largest key) are settled
// up front and the digits start right below them, so keys from a narrow score
// range spread over many bins.  Otherwise the digits are bits 31-21, 20-10
// and 9-0.
template <int NT, bool Adaptive, class ForKeys>
__device__ uint32_t radix_cut(ForKeys for_keys, uint32_t kk, uint32_t* hist, uint64_t* sh_scan, uint32_t* sh_cut,
                              uint32_t* take_eq) {
  constexpr int kBPT = kBins / NT;  // consecutive bins owned by one thread in the scan
  constexpr int kW = NT / kWave;
  static_assert(kBins % NT == 0, "bins split evenly");
  int common = 0;  // leading bits shared by every key
  uint32_t kmin = 0u;
  if constexpr (Adaptive) {
    kmin = 0xffffffffu;
    uint32_t kmax = 0u;
    for_keys([&](uint32_t key) {
      kmin = min(kmin, key);
      kmax = max(kmax, key);
    });
    kmin = wave_incl_scan_op(kmin, 0xffffffffu, [](uint32_t a, uint32_t b) { return min(a, b); });
    kmax = wave_incl_scan_op(kmax, 0u, [](uint32_t a, uint32_t b) { return max(a, b); });
    uint32_t* sh_mm = reinterpret_cast<uint32_t*>(sh_scan);  // [kW] minima, [kW] maxima
    if ((threadIdx.x & (kWave - 1)) == kWave - 1) {
      sh_mm[threadIdx.x / kWave] = kmin;
      sh_mm[kW + threadIdx.x / kWave] = kmax;
    }
    __syncthreads();
    kmin = sh_mm[0];
    kmax = sh_mm[kW];
#pragma unroll
    for (int w = 1; w < kW; ++w) {
      kmin = min(kmin, sh_mm[w]);
      kmax = max(kmax, sh_mm[kW + w]);
    }
    __syncthreads();
    common = kmin == kmax ? 32 : __clz(kmin ^ kmax);  // 0..32
  }
  uint32_t pmask = static_cast<uint32_t>(0xffffffff00000000ull >> common);  // top `common` bits
  uint32_t prefix = kmin & pmask;
  int sh = 32 - common;  // bits below the prefix still to settle (at most 3 passes of <= 11)
#pragma unroll 1
  while (sh > 0) {
    const int w = sh < 11 ? sh : 11;
    sh -= w;
    const uint32_t dm = (1u << w) - 1u;
    for (int b = threadIdx.x; b < kCopies * kBins; b += NT) hist[b] = 0u;
    __syncthreads();
    uint32_t* my_hist = hist + (threadIdx.x % kCopies) * kBins;
    for_keys([&](uint32_t key) {
      if ((key & pmask) == prefix) atomicAdd(&my_hist[(key >> sh) & dm], 1u);
    });
    __syncthreads();
    const int nb = static_cast<int>(dm) + 1;
    const int b0 = kBPT * threadIdx.x;
    uint32_t c[kBPT];
    uint32_t mine = 0u;
#pragma unroll
    for (int j = 0; j < kBPT; ++j) {
      c[j] = 0u;
      if (b0 + j < nb) {
#pragma unroll
        for (int cp = 0; cp < kCopies; ++cp) c[j] += hist[cp * kBins + b0 + j];
      }
      mine += c[j];
    }
    uint64_t tot;
    const uint64_t excl = block_excl_scan<NT>(mine, sh_scan, tot);  // keys in bins below b0
    // Keys strictly above bin b0 + j = total - (keys in bins <= b0 + j); the
    // cut bin b satisfies above(b) < kk <= above(b) + count(b).
    uint32_t upto = static_cast<uint32_t>(excl);
#pragma unroll
    for (int j = 0; j < kBPT; ++j) {
      upto += c[j];
      const uint32_t above = static_cast<uint32_t>(tot) - upto;
      if (b0 + j < nb && above < kk && kk <= above + c[j]) {
        sh_cut[0] = static_cast<uint32_t>(b0 + j);
        sh_cut[1] = kk - above;
      }
    }
    __syncthreads();
    const uint32_t bin = sh_cut[0];
    kk = sh_cut[1];
    prefix |= bin << sh;
    pmask |= dm << sh;
    __syncthreads();
  }
  *take_eq = kk;
  return prefix;
}

// Keys of one score row read from global memory on every pass, kU loads in
// flight per thread before any of them is used.
template <int NT>
struct RowKeys {
  static constexpr int kU = 16;
  const float* row;
  int n;
  template <class F>
  __device__ __forceinline__ void operator()(F&& f) const {
    int i = threadIdx.x;
    for (; i + (kU - 1) * NT < n; i += kU * NT) {
      float v[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) v[u] = row[i + u * NT];
#pragma unroll
      for (int u = 0; u < kU; ++u) f(score_key(v[u]));
    }
    for (; i < n; i += NT) f(score_key(row[i]));
  }
};

// Emit, in ascending position order, every i with key > cut plus the first
// `take_eq` positions with key == cut, as first + i, or out_map[i] when
// out_map != nullptr.  Writes stop at cap entries.
template <int NT>
__device__ void emit_selected(const float* __restrict__ row, int n, uint32_t cut, uint32_t take_eq,
                              const int32_t* __restrict__ out_map, int first, int32_t* __restrict__ out,
                              uint32_t cap, uint64_t* sh_scan) {
  constexpr int E = 8;  // consecutive elements per thread per chunk
  uint32_t eq_before = 0u, sel_before = 0u;
  for (int base = 0; base < n; base += NT * E) {
    const int i0 = base + threadIdx.x * E;
    uint32_t gt = 0u, eq = 0u;
    uint32_t flags = 0u;  // bit e: gt, bit 8+e: eq
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int i = i0 + e;
      if (i < n) {
        const uint32_t key = score_key(row[i]);
        if (key > cut) { ++gt; flags |= 1u << e; }
        else if (key == cut) { ++eq; flags |= 1u << (8 + e); }
      }
    }
    uint64_t tot;
    const uint64_t mine = (static_cast<uint64_t>(gt) << 32) | eq;
    const uint64_t excl = block_excl_scan<NT>(mine, sh_scan, tot);
    uint32_t eq_rank = eq_before + static_cast<uint32_t>(excl & 0xffffffffu);
    const uint32_t gt_rank = static_cast<uint32_t>(excl >> 32);
    uint32_t eq_taken_before = eq_rank < take_eq ? eq_rank : take_eq;
    uint32_t o = sel_before + gt_rank + (eq_taken_before - (eq_before < take_eq ? eq_before : take_eq));
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int i = i0 + e;
      bool take = false;
      if (flags & (1u << e)) take = true;
      else if (flags & (1u << (8 + e))) { take = eq_rank < take_eq; ++eq_rank; }
      if (take) {
        if (o < cap) out[o] = out_map ? out_map[i] : first + i;
        ++o;
      }
    }
    const uint32_t tot_gt = static_cast<uint32_t>(tot >> 32);
    const uint32_t tot_eq = static_cast<uint32_t>(tot & 0xffffffffu);
    const uint32_t eq_after = eq_before + tot_eq;
    const uint32_t took = (eq_after < take_eq ? eq_after : take_eq) - (eq_before < take_eq ? eq_before : take_eq);
    sel_before += tot_gt + took;
    eq_before = eq_after;
  }
}

// Row b of the selection.  Fixed rows: n_row scores at b * n_row, k_total
// outputs at b * k_total, positions 0..n_row-1.  Ragged rows (packed samples):
// scores cu_n[b] .. cu_n[b+1]-1, outputs cu_k[b] .. cu_k[b+1]-1, and the
// written positions are packed row indices (cu_n[b] + local position).  A
// ragged row asks for at most its length and at least its forced ends; counts
// outside that are clamped (the unused outputs are left untouched).
struct SelRow {
  int64_t in_off, out_off;
  int n, k, f, l, base;
  __device__ __forceinline__ SelRow(int64_t b, int n_row, int k_total, int f_, int l_, const int32_t* cu_n,
                                    const int32_t* cu_k) {
    if (cu_n) {  // n_row / k_total are then the packed score count / output capacity; rows are clamped into them
      in_off = min(max(cu_n[b], 0), n_row);
      n = max(0, min(cu_n[b + 1], n_row) - static_cast<int>(in_off));
      out_off = min(max(cu_k[b], 0), k_total);
      k = max(0, min(min(cu_k[b + 1] - cu_k[b], n), k_total - static_cast<int>(out_off)));
      f = min(f_, k);
      l = min(l_, k - f);
      base = static_cast<int>(in_off);
    } else {
      in_off = b * n_row;
      n = n_row;
      out_off = b * k_total;
      k = k_total;
      f = f_;
      l = l_;
      base = 0;
    }
  }
};

// Forced retention: the first f and last l positions of a row of n_row
// scores are written to the two ends of its k_total outputs; the caller then
// selects k_total - f - l among the middle positions.
template <int NT>
__device__ __forceinline__ void emit_forced(int n_row, int k_total, int f, int l, const int32_t* __restrict__ pos,
                                            int base, int32_t* __restrict__ out) {
  for (int i = threadIdx.x; i < f; i += NT) out[i] = pos ? pos[i] : base + i;
  for (int j = threadIdx.x; j < l; j += NT) {
    const int i = n_row - l + j;
    out[k_total - l + j] = pos ? pos[i] : base + i;
  }
}

// Rows of any length: keys are re-read from global memory on every pass
// (Adaptive: one more read settles the common key prefix first; worth it for a
// single row, where same-bin atomics dominate, not for batches).
template <int NT, bool Adaptive>
__global__ __launch_bounds__(NT, 1)
void topk_kernel(const float* __restrict__ score, int n_row, int k_total, int f_in, int l_in,
                 const int32_t* __restrict__ pos, int32_t* __restrict__ idx, const int32_t* __restrict__ cu_n,
                 const int32_t* __restrict__ cu_k) {
  __shared__ uint32_t hist[kCopies * kBins];
  __shared__ uint64_t sh_scan[2 * (NT / kWave) + 8];
  __shared__ uint32_t sh_cut[2];
  const SelRow rw(blockIdx.x, n_row, k_total, f_in, l_in, cu_n, cu_k);
  const int f = rw.f, l = rw.l;
  int32_t* out = idx + rw.out_off;
  emit_forced<NT>(rw.n, rw.k, f, l, pos, rw.base, out);
  const int n = rw.n - f - l;
  const int k = rw.k - f - l;
  if (k <= 0) return;
  const float* r = score + rw.in_off + f;
  uint32_t take_eq;
  const uint32_t cut =
      radix_cut<NT, Adaptive>(RowKeys<NT>{r, n}, static_cast<uint32_t>(k), hist, sh_scan, sh_cut, &take_eq);
  emit_selected<NT>(r, n, cut, take_eq, pos ? pos + f : nullptr, rw.base + f, out + f, static_cast<uint32_t>(k),
                   sh_scan);
}

// Rows of up to NT * ITEMS scores: each thread loads its ITEMS consecutive
// scores once, keeps their keys in registers for the three radix passes, and
// emits its survivors after one workgroup scan (thread order is position
// order).
template <int NT, int ITEMS>
__global__ __launch_bounds__(NT, 1)
void topk_reg_kernel(const float* __restrict__ score, int n_row, int k_total, int f_in, int l_in,
                     const int32_t* __restrict__ pos, int32_t* __restrict__ idx, const int32_t* __restrict__ cu_n,
                     const int32_t* __restrict__ cu_k) {
  static_assert(ITEMS <= 32, "masks are 32-bit");
  __shared__ uint32_t hist[kCopies * kBins];
  __shared__ uint64_t sh_scan[2 * (NT / kWave) + 8];
  __shared__ uint32_t sh_cut[2];
  const SelRow rw(blockIdx.x, n_row, k_total, f_in, l_in, cu_n, cu_k);
  const int f = rw.f, l = rw.l;
  int32_t* out = idx + rw.out_off;
  emit_forced<NT>(rw.n, rw.k, f, l, pos, rw.base, out);
  const int n = min(rw.n - f - l, NT * ITEMS);  // rows longer than the launch assumed are cut (never read past)
  const int k = rw.k - f - l;
  if (k <= 0) return;
  const float* r = score + rw.in_off + f;
  out += f;
  const int i0 = threadIdx.x * ITEMS;
  uint32_t keys[ITEMS];
#pragma unroll
  for (int e = 0; e < ITEMS; ++e) keys[e] = (i0 + e < n) ? score_key(r[i0 + e]) : 0u;
  const int valid = n - i0;  // keys e < valid exist
  auto for_keys = [&](auto&& fn) {
#pragma unroll
    for (int e = 0; e < ITEMS; ++e)
      if (e < valid) fn(keys[e]);
  };
  uint32_t take_eq;
  const uint32_t cut = radix_cut<NT, true>(for_keys, static_cast<uint32_t>(k), hist, sh_scan, sh_cut, &take_eq);
  uint32_t gt_mask = 0u, eq_mask = 0u;
#pragma unroll
  for (int e = 0; e < ITEMS; ++e) {
    if (e < valid) {
      if (keys[e] > cut) gt_mask |= 1u << e;
      else if (keys[e] == cut) eq_mask |= 1u << e;
    }
  }
  const uint32_t gt = __popc(gt_mask), eq = __popc(eq_mask);
  uint64_t tot;
  const uint64_t excl = block_excl_scan<NT>((static_cast<uint64_t>(gt) << 32) | eq, sh_scan, tot);
  uint32_t eq_rank = static_cast<uint32_t>(excl & 0xffffffffu);
  uint32_t o = static_cast<uint32_t>(excl >> 32) + (eq_rank < take_eq ? eq_rank : take_eq);
#pragma unroll
  for (int e = 0; e < ITEMS; ++e) {
    bool take = (gt_mask >> e) & 1u;
    if ((eq_mask >> e) & 1u) { take = eq_rank < take_eq; ++eq_rank; }
    if (take) {
      if (o < static_cast<uint32_t>(k)) out[o] = pos ? pos[f + i0 + e] : rw.base + f + i0 + e;
      ++o;
    }
  }
}

__global__ __launch_bounds__(kSelThreads, 1)
void order_stat_kernel(const float* __restrict__ score, const int32_t* __restrict__ n_dev, int n_max,
                       int rank, float* __restrict__ tau_out) {
  __shared__ uint32_t hist[kCopies * kBins];
  __shared__ uint64_t sh_scan[2 * kSelWaves + 8];
  __shared__ uint32_t sh_cut[2];
  int n = n_dev ? *n_dev : n_max;
  if (n > n_max) n = n_max;
  if (rank < 1 || rank > n) {
    if (threadIdx.x == 0) *tau_out = __uint_as_float(0x7fc00000u);
    return;
  }
  uint32_t take_eq;
  // rank-th smallest == (n - rank + 1)-th largest under the same total order.
  const uint32_t cut = radix_cut<kSelThreads, true>(RowKeys<kSelThreads>{score, n},
                                                     static_cast<uint32_t>(n - rank + 1), hist, sh_scan, sh_cut,
                                                     &take_eq);
  if (threadIdx.x == 0) *tau_out = key_score(cut);
}

__global__ __launch_bounds__(kSelThreads, 1)
void threshold_kernel(const float* __restrict__ score, const int32_t* __restrict__ pos,
                      const int32_t* __restrict__ n_dev, int n_max, const float* __restrict__ tau_p,
                      int patience, uint8_t* __restrict__ counters, int32_t* __restrict__ out,
                      int32_t* __restrict__ n_out) {
  __shared__ uint64_t sh_scan[2 * kSelWaves + 8];
  int n = n_dev ? *n_dev : n_max;
  if (n > n_max) n = n_max;
  if (n < 0) n = 0;
  const float tau = *tau_p;
  constexpr int E = 16;  // consecutive rows per thread per chunk; all loads issued before use
  uint32_t before = 0u;
  for (int base = 0; base < n; base += kSelThreads * E) {
    const int i0 = base + threadIdx.x * E;
    uint32_t keep_bits = 0u, cnt = 0u;
    int32_t p[E];
    float sc[E];
    uint8_t c0[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int i = i0 + e;
      p[e] = i < n ? (pos ? pos[i] : i) : -1;
      sc[e] = i < n ? score[i] : 0.f;
    }
#pragma unroll
    for (int e = 0; e < E; ++e) c0[e] = p[e] >= 0 ? counters[p[e]] : 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if (p[e] >= 0) {
        const uint32_t c = (sc[e] < tau) ? static_cast<uint32_t>(c0[e]) + 1u : 0u;
        counters[p[e]] = static_cast<uint8_t>(c > 255u ? 255u : c);
        if (c < static_cast<uint32_t>(patience)) { keep_bits |= 1u << e; ++cnt; }
      }
    }
    uint64_t tot;
    const uint64_t excl = block_excl_scan<kSelThreads>(cnt, sh_scan, tot);
    uint32_t o = before + static_cast<uint32_t>(excl);
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (keep_bits & (1u << e)) {
        if (o < static_cast<uint32_t>(n_max)) out[o] = p[e];  // never beyond the capacity
        ++o;
      }
    before += static_cast<uint32_t>(tot);
  }
  if (threadIdx.x == 0) *n_out = static_cast<int32_t>(before);
}

}  // namespace

namespace {

// ---------------------------------------------------------------------------
// Batched rows: one wave per row, no workgroup barrier anywhere.  Lane l holds
// the keys of positions 256*j + 4*l + e (e < 4, j < J) in registers (one
// 16-byte load each), counts into its wave's own 2048-bin LDS histogram, and
// settles the cut with wave scans; the emit walks the 256-position chunks in
// order with one scan each.  Rows are n % 4 == 0 scores, 16-byte aligned.
// ---------------------------------------------------------------------------
constexpr int kWaveRowsPerBlock = 4;

__device__ __forceinline__ void wave_lds_fence() { __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront"); }

template <int J>
__global__ __launch_bounds__(kWaveRowsPerBlock * kWave)
void topk_wave_kernel(const float* __restrict__ score, int rows, int n, int k, int32_t* __restrict__ idx) {
  __shared__ uint32_t hist_all[kWaveRowsPerBlock * kBins];
  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x / kWave;
  const int row = blockIdx.x * kWaveRowsPerBlock + w;
  if (row >= rows) return;  // the whole wave leaves; nothing below synchronises waves
  uint32_t* h = hist_all + w * kBins;
  const u32x4* r4 = reinterpret_cast<const u32x4*>(score + static_cast<size_t>(row) * n);
  int32_t* out = idx + static_cast<size_t>(row) * k;
  const int n4 = n >> 2;
  uint32_t keys[J][4];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int i4 = j * kWave + lane;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (i4 < n4) v = __builtin_nontemporal_load(r4 + i4);
#pragma unroll
    for (int e = 0; e < 4; ++e) keys[j][e] = score_key(__uint_as_float(v[e]));
  }
  auto valid = [&](int j) { return j * kWave + lane < n4; };

  // Bits shared by every key of the row are settled first (wave min/max of the
  // keys in registers); digits of up to 11 bits then start right below them, so
  // a narrow score range spreads over many bins instead of piling same-address
  // atomics onto a few.  (Widths are computed, not looked up: a table would put
  // scalar loads on the counter the LDS atomics use.)
  uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    if (valid(j)) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kmin = min(kmin, keys[j][e]);
        kmax = max(kmax, keys[j][e]);
      }
    }
  }
  kmin = wave_incl_scan_op(kmin, 0xffffffffu, [](uint32_t a, uint32_t b) { return min(a, b); });
  kmax = wave_incl_scan_op(kmax, 0u, [](uint32_t a, uint32_t b) { return max(a, b); });
  kmin = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(kmin), kWave - 1));
  kmax = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(kmax), kWave - 1));
  const int common = kmin == kmax ? 32 : __clz(kmin ^ kmax);
  uint32_t pmask = static_cast<uint32_t>(0xffffffff00000000ull >> common);
  uint32_t prefix = kmin & pmask, kk = static_cast<uint32_t>(k);
  constexpr int kBPL = kBins / kWave;  // bins per lane in the scan (32)
  int sh = 32 - common;
#pragma unroll 1
  while (sh > 0) {
    const int wd = sh < 11 ? sh : 11;
    sh -= wd;
    const uint32_t dm = (1u << wd) - 1u;
#pragma unroll
    for (int b = 0; b < kBPL; ++b) h[b * kWave + lane] = 0u;
    wave_lds_fence();
#pragma unroll
    for (int j = 0; j < J; ++j) {
      if (valid(j)) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if ((keys[j][e] & pmask) == prefix) atomicAdd(&h[(keys[j][e] >> sh) & dm], 1u);
      }
    }
    wave_lds_fence();
    const int nb = static_cast<int>(dm) + 1;
    const int b0 = lane * kBPL;
    uint32_t c[kBPL];
    uint32_t mine = 0u;
#pragma unroll
    for (int b = 0; b < kBPL; ++b) {
      c[b] = (b0 + b < nb) ? h[b0 + b] : 0u;
      mine += c[b];
    }
    const uint32_t incl = wave_incl_scan32(mine);
    const uint32_t tot = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(incl), kWave - 1));
    uint32_t upto = incl - mine;  // keys in bins below b0
    uint32_t found_bin = 0u, found_kk = 0u;
    bool found = false;
#pragma unroll
    for (int b = 0; b < kBPL; ++b) {
      upto += c[b];
      const uint32_t above = tot - upto;  // keys in bins above b0 + b
      if (b0 + b < nb && above < kk && kk <= above + c[b]) {
        found = true;
        found_bin = static_cast<uint32_t>(b0 + b);
        found_kk = kk - above;
      }
    }
    const uint64_t who = __ballot(found);
    const int src = static_cast<int>(__builtin_ctzll(who));
    const uint32_t bin = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(found_bin), src));
    kk = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(found_kk), src));
    prefix |= bin << sh;
    pmask |= dm << sh;
  }
  const uint32_t cut = prefix, take_eq = kk;

  // Emit in position order: chunk j covers positions 256*j .. 256*j + 255, lane
  // l its four positions 256*j + 4*l + e.
  uint32_t sel_before = 0u, eq_before = 0u;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    uint32_t gt_bits = 0u, eq_bits = 0u;
    if (valid(j)) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (keys[j][e] > cut) gt_bits |= 1u << e;
        else if (keys[j][e] == cut) eq_bits |= 1u << e;
      }
    }
    const uint32_t packed = (static_cast<uint32_t>(__popc(gt_bits)) << 16) | static_cast<uint32_t>(__popc(eq_bits));
    const uint32_t incl = wave_incl_scan32(packed);  // per-chunk sums stay below 2^16
    const uint32_t tot = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(incl), kWave - 1));
    const uint32_t excl = incl - packed;
    uint32_t eq_rank = eq_before + (excl & 0xffffu);
    const uint32_t taken_eq_before = min(eq_rank, take_eq) - min(eq_before, take_eq);
    uint32_t o = sel_before + (excl >> 16) + taken_eq_before;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      bool take = (gt_bits >> e) & 1u;
      if ((eq_bits >> e) & 1u) { take = eq_rank < take_eq; ++eq_rank; }
      if (take) {
        if (o < static_cast<uint32_t>(k)) out[o] = j * 4 * kWave + 4 * lane + e;
        ++o;
      }
    }
    const uint32_t tot_eq = tot & 0xffffu;
    sel_before += (tot >> 16) + (min(eq_before + tot_eq, take_eq) - min(eq_before, take_eq));
    eq_before += tot_eq;
  }
}

// n: the row length (ragged: the packed score count); n_longest: the longest
// row (picks the kernel); cu_n / cu_k: ragged layout or null.
template <int NT>
void launch_topk_nt(const float* score, int rows, int n, int k, int f, int l, const int32_t* pos, int32_t* idx,
                    const int32_t* cu_n, const int32_t* cu_k, hipStream_t stream, int n_longest = -1) {
  const int n_mid = cu_n ? n_longest : n - f - l;
  const dim3 g(rows), b(NT);
  if (n_mid <= NT * 4)
    hipLaunchKernelGGL((topk_reg_kernel<NT, 4>), g, b, 0, stream, score, n, k, f, l, pos, idx, cu_n, cu_k);
  else if (n_mid <= NT * 8)
    hipLaunchKernelGGL((topk_reg_kernel<NT, 8>), g, b, 0, stream, score, n, k, f, l, pos, idx, cu_n, cu_k);
  else if (n_mid <= NT * 16)
    hipLaunchKernelGGL((topk_reg_kernel<NT, 16>), g, b, 0, stream, score, n, k, f, l, pos, idx, cu_n, cu_k);
  else if (n_mid <= NT * 32)
    hipLaunchKernelGGL((topk_reg_kernel<NT, 32>), g, b, 0, stream, score, n, k, f, l, pos, idx, cu_n, cu_k);
  else if (rows == 1)
    hipLaunchKernelGGL((topk_kernel<NT, true>), g, b, 0, stream, score, n, k, f, l, pos, idx, cu_n, cu_k);
  else
    hipLaunchKernelGGL((topk_kernel<NT, false>), g, b, 0, stream, score, n, k, f, l, pos, idx, cu_n, cu_k);
}

}  // namespace

// Many rows of at most 8192 aligned scores without forced ends or a position
// map: one wave per row.  Otherwise one 1024-thread workgroup per row.
hipError_t launch_topk(const float* score, int rows, int n, int k, int keep_first, int keep_last,
                       const int32_t* pos, int32_t* idx, hipStream_t stream) {
  if (rows == 0 || k == 0) return hipSuccess;
  const bool wave_rows = rows >= kWaveRowsMin && !pos && keep_first == 0 && keep_last == 0 && n % 4 == 0 &&
                         n <= 8192 && (reinterpret_cast<uintptr_t>(score) & 15u) == 0;
  if (wave_rows) {
    const dim3 grid((rows + kWaveRowsPerBlock - 1) / kWaveRowsPerBlock), block(kWaveRowsPerBlock * kWave);
    if (n <= 2048)
      hipLaunchKernelGGL(topk_wave_kernel<8>, grid, block, 0, stream, score, rows, n, k, idx);
    else if (n <= 4096)
      hipLaunchKernelGGL(topk_wave_kernel<16>, grid, block, 0, stream, score, rows, n, k, idx);
    else
      hipLaunchKernelGGL(topk_wave_kernel<32>, grid, block, 0, stream, score, rows, n, k, idx);
  } else {
    launch_topk_nt<kSelThreads>(score, rows, n, k, keep_first, keep_last, pos, idx, nullptr, nullptr, stream);
  }
  return hipGetLastError();
}

hipError_t launch_topk_ragged(const float* score, int n_total, int B, const int32_t* cu_n, const int32_t* cu_k,
                              int max_n, int k_cap, int keep_first, int keep_last, int32_t* idx, hipStream_t stream) {
  if (B == 0 || max_n == 0 || k_cap == 0 || n_total == 0) return hipSuccess;
  launch_topk_nt<kSelThreads>(score, B, n_total, k_cap, keep_first, keep_last, nullptr, idx, cu_n, cu_k, stream,
                              max_n);
  return hipGetLastError();
}

hipError_t launch_order_stat(const float* score, const int32_t* n_dev, int n_max, int rank, float* tau_out,
                             hipStream_t stream) {
  hipLaunchKernelGGL(order_stat_kernel, dim3(1), dim3(kSelThreads), 0, stream, score, n_dev, n_max, rank,
                     tau_out);
  return hipGetLastError();
}

hipError_t launch_threshold(const float* score, const int32_t* pos, const int32_t* n_dev, int n_max,
                            const float* tau, int patience, uint8_t* counters, int32_t* out,
                            int32_t* n_out, hipStream_t stream) {
  hipLaunchKernelGGL(threshold_kernel, dim3(1), dim3(kSelThreads), 0, stream, score, pos, n_dev, n_max, tau,
                     patience, counters, out, n_out);
  return hipGetLastError();
}

}  // namespace dash
