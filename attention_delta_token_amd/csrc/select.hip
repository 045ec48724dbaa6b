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
// 256 rows of at most 8192 aligned scores take one wave per row instead, and
// rows of more than 2048 of those bracket the cut from a sample first).
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
// `nan` accumulates this thread's count of NaN scores (key 0).
template <int NT>
__device__ void emit_selected(const float* __restrict__ row, int n, uint32_t cut, uint32_t take_eq,
                              const int32_t* __restrict__ out_map, int first, int32_t* __restrict__ out,
                              uint32_t cap, uint64_t* sh_scan, uint32_t& nan) {
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
        nan += key == 0u;
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
// outputs at b * k_total, positions 0..n_row-1; with a device count (one row),
// the row holds min(*n_dev, n_row) scores and keeps at most that many.  Ragged
// rows (packed samples): scores cu_n[b] .. cu_n[b+1]-1, outputs cu_k[b] ..
// cu_k[b+1]-1, and the written positions are packed row indices (cu_n[b] +
// local position).  A row asks for at most its length and at least its forced
// ends; counts outside that are clamped (the unused outputs are left
// untouched).
struct SelRow {
  int64_t in_off, out_off;
  int n, k, f, l, base;
  __device__ __forceinline__ SelRow(int64_t b, int n_row, int k_total, int f_, int l_, const int32_t* cu_n,
                                    const int32_t* cu_k, const int32_t* n_dev) {
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
      out_off = b * k_total;
      base = 0;
      if (n_dev) {
        n = min(max(*n_dev, 0), n_row);
        k = min(k_total, n);
        f = min(f_, k);
        l = min(l_, k - f);
      } else {
        n = n_row;
        k = k_total;
        f = f_;
        l = l_;
      }
    }
  }
};

// NaN scores among the forced ends of a row (positions 0..f-1 and n-l..n-1),
// this thread's share.
template <int NT>
__device__ __forceinline__ uint32_t forced_nans(const float* __restrict__ row, int n, int f, int l) {
  uint32_t c = 0u;
  for (int i = threadIdx.x; i < f; i += NT) c += score_key(row[i]) == 0u;
  for (int j = threadIdx.x; j < l; j += NT) c += score_key(row[n - l + j]) == 0u;
  return c;
}

// Workgroup total of a per-thread count, written by thread 0 to *out.
template <int NT>
__device__ __forceinline__ void write_block_total(uint32_t mine, uint64_t* sh_scan, int32_t* out) {
  uint64_t tot;
  (void)block_excl_scan<NT>(mine, sh_scan, tot);
  if (threadIdx.x == 0) *out = static_cast<int32_t>(tot);
}

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
                 const int32_t* __restrict__ cu_k, const int32_t* __restrict__ n_dev, int32_t* __restrict__ n_out,
                 int32_t* __restrict__ nan_out) {
  __shared__ uint32_t hist[kCopies * kBins];
  __shared__ uint64_t sh_scan[2 * (NT / kWave) + 8];
  __shared__ uint32_t sh_cut[2];
  const SelRow rw(blockIdx.x, n_row, k_total, f_in, l_in, cu_n, cu_k, n_dev);
  const int f = rw.f, l = rw.l;
  int32_t* out = idx + rw.out_off;
  if (n_out && threadIdx.x == 0) *n_out = rw.k;
  emit_forced<NT>(rw.n, rw.k, f, l, pos, rw.base, out);
  const int n = rw.n - f - l;
  const int k = rw.k - f - l;
  const float* r = score + rw.in_off + f;
  uint32_t nan = nan_out ? forced_nans<NT>(score + rw.in_off, rw.n, f, l) : 0u;
  if (k <= 0) {
    if (nan_out) {
      for (int i = threadIdx.x; i < n; i += NT) nan += score_key(r[i]) == 0u;
      write_block_total<NT>(nan, sh_scan, nan_out + blockIdx.x);
    }
    return;
  }
  uint32_t take_eq;
  const uint32_t cut =
      radix_cut<NT, Adaptive>(RowKeys<NT>{r, n}, static_cast<uint32_t>(k), hist, sh_scan, sh_cut, &take_eq);
  emit_selected<NT>(r, n, cut, take_eq, pos ? pos + f : nullptr, rw.base + f, out + f, static_cast<uint32_t>(k),
                   sh_scan, nan);
  if (nan_out) write_block_total<NT>(nan, sh_scan, nan_out + blockIdx.x);
}

// Rows of up to NT * ITEMS scores: each thread loads its ITEMS consecutive
// scores once, keeps their keys in registers for the three radix passes, and
// emits its survivors after one workgroup scan (thread order is position
// order).
template <int NT, int ITEMS>
__global__ __launch_bounds__(NT, 1)
void topk_reg_kernel(const float* __restrict__ score, int n_row, int k_total, int f_in, int l_in,
                     const int32_t* __restrict__ pos, int32_t* __restrict__ idx, const int32_t* __restrict__ cu_n,
                     const int32_t* __restrict__ cu_k, const int32_t* __restrict__ n_dev,
                     int32_t* __restrict__ n_out, int32_t* __restrict__ nan_out) {
  static_assert(ITEMS <= 32, "masks are 32-bit");
  using Mask = uint32_t;
  __shared__ uint32_t hist[kCopies * kBins];
  __shared__ uint64_t sh_scan[2 * (NT / kWave) + 8];
  __shared__ uint32_t sh_cut[2];
  const SelRow rw(blockIdx.x, n_row, k_total, f_in, l_in, cu_n, cu_k, n_dev);
  const int f = rw.f, l = rw.l;
  int32_t* out = idx + rw.out_off;
  if (n_out && threadIdx.x == 0) *n_out = rw.k;
  emit_forced<NT>(rw.n, rw.k, f, l, pos, rw.base, out);
  const int n = min(rw.n - f - l, NT * ITEMS);  // rows longer than the launch assumed are cut (never read past)
  const int k = rw.k - f - l;
  const float* r = score + rw.in_off + f;
  out += f;
  const int i0 = threadIdx.x * ITEMS;
  uint32_t keys[ITEMS];
#pragma unroll
  for (int e = 0; e < ITEMS; ++e) keys[e] = 0u;
  if (n > 0) {
    // every load unconditional (positions past the row re-read its last
    // score; they are excluded through `valid` below), so all are in flight
    // before the first is used
#pragma unroll
    for (int e = 0; e < ITEMS; ++e) keys[e] = __float_as_uint(r[min(i0 + e, n - 1)]);
#pragma unroll
    for (int e = 0; e < ITEMS; ++e) keys[e] = score_key(__uint_as_float(keys[e]));
  }
  const int valid = n - i0;  // keys e < valid exist
  uint32_t nan = 0u;
  if (nan_out) {
    nan = forced_nans<NT>(score + rw.in_off, rw.n, f, l);
#pragma unroll
    for (int e = 0; e < ITEMS; ++e) nan += (e < valid && keys[e] == 0u) ? 1u : 0u;
  }
  if (k <= 0) {
    if (nan_out) write_block_total<NT>(nan, sh_scan, nan_out + blockIdx.x);
    return;
  }
  auto for_keys = [&](auto&& fn) {
    // `valid` made opaque at every call: the per-item tests stay next to
    // their use instead of being kept as one compare mask per item across
    // the radix passes (scalar-register pressure)
    int vld = valid;
    asm volatile("" : "+v"(vld));
#pragma unroll
    for (int e = 0; e < ITEMS; ++e)
      if (e < vld) fn(keys[e]);
  };
  uint32_t take_eq;
  const uint32_t cut = radix_cut<NT, true>(for_keys, static_cast<uint32_t>(k), hist, sh_scan, sh_cut, &take_eq);
  Mask gt_mask = 0u, eq_mask = 0u;
#pragma unroll
  for (int e = 0; e < ITEMS; ++e) {
    if (e < valid) {
      if (keys[e] > cut) gt_mask |= Mask(1) << e;
      else if (keys[e] == cut) eq_mask |= Mask(1) << e;
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
  if (nan_out) write_block_total<NT>(nan, sh_scan, nan_out + blockIdx.x);
}

// Batched rows of up to 64 keys per thread (NT threads, C chunks), plain rows
// only (no forced ends, position map or device count; n % 4 == 0, 16-byte
// aligned): chunk c of a row is positions 4 (c NT + t) + q, so every load of
// a chunk is one coalesced 16-byte load per thread and the whole row sits in
// registers for the radix passes.  The emit counts, per chunk and thread, the
// keys above the cut and equal to it; a workgroup scan of those counts per
// chunk (wave scans, then the waves' totals in wave order inside a chunk and
// the chunks' totals in chunk order) gives every kept key its output slot in
// ascending position order, ties to the lower position.
template <int NT, int C>
__global__ __launch_bounds__(NT, 1)
void topk_strided_kernel(const float* __restrict__ score, int n, int k, int32_t* __restrict__ idx,
                         int32_t* __restrict__ nan_out) {
  constexpr int kW = NT / kWave;
  static_assert(C <= kWave, "one lane per chunk in the base scan");
  __shared__ uint32_t hist[kCopies * kBins];
  __shared__ uint64_t sh_scan[2 * kW + 8];
  __shared__ uint32_t sh_cut[2];
  __shared__ uint32_t sh_tot[kW][C];    // per wave and chunk: (greater << 16) | equal
  __shared__ uint32_t sh_wbase[kW][C];  // the same, summed over the lower waves of the chunk
  __shared__ uint32_t sh_cbase[2][C];   // greater / equal keys in all lower chunks
  const int t = threadIdx.x, lane = t & (kWave - 1), wave = t / kWave;
  const u32x4* r4 = reinterpret_cast<const u32x4*>(score + static_cast<size_t>(blockIdx.x) * n);
  int32_t* out = idx + static_cast<size_t>(blockIdx.x) * k;
  const int n4 = n >> 2;
  uint32_t keys[C][4];
#pragma unroll
  for (int c = 0; c < C; ++c) {  // unconditional loads, all in flight before the first use
    const u32x4 v = __builtin_nontemporal_load(r4 + min(c * NT + t, n4 - 1));
#pragma unroll
    for (int q = 0; q < 4; ++q) keys[c][q] = v[q];
  }
#pragma unroll
  for (int c = 0; c < C; ++c)
#pragma unroll
    for (int q = 0; q < 4; ++q) keys[c][q] = score_key(__uint_as_float(keys[c][q]));
  const int vld_n = n4 - t;  // chunk c of this thread exists iff c NT < vld_n
  uint32_t nan = 0u;
  if (nan_out) {
#pragma unroll
    for (int c = 0; c < C; ++c)
#pragma unroll
      for (int q = 0; q < 4; ++q) nan += (c * NT < vld_n && keys[c][q] == 0u) ? 1u : 0u;
  }
  if (k > 0) {
    auto for_keys = [&](auto&& fn) {
      int vld = vld_n;  // opaque at every call: the chunk tests stay next to their use
      asm volatile("" : "+v"(vld));
#pragma unroll
      for (int c = 0; c < C; ++c)
        if (c * NT < vld)
#pragma unroll
          for (int q = 0; q < 4; ++q) fn(keys[c][q]);
    };
    uint32_t take_eq;
    const uint32_t cut = radix_cut<NT, true>(for_keys, static_cast<uint32_t>(k), hist, sh_scan, sh_cut, &take_eq);
    auto counts = [&](int c) {  // (greater << 16) | equal over this thread's four keys of chunk c
      uint32_t gt = 0u, eq = 0u;
      if (c * NT < vld_n) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          gt += keys[c][q] > cut ? 1u : 0u;
          eq += keys[c][q] == cut ? 1u : 0u;
        }
      }
      return (gt << 16) | eq;
    };
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const uint32_t incl = wave_incl_scan32(counts(c));  // fields stay below 2^16 (256 per wave)
      if (lane == kWave - 1) sh_tot[wave][c] = incl;
    }
    __syncthreads();
    if (wave == 0) {
      uint32_t gt = 0u, eq = 0u;  // lane c: chunk c, its waves in order
      if (lane < C) {
        uint32_t run = 0u;
        for (int w = 0; w < kW; ++w) {
          sh_wbase[w][lane] = run;
          run += sh_tot[w][lane];  // per chunk at most NT * 4 = 4096 per field
        }
        gt = run >> 16;
        eq = run & 0xffffu;
      }
      const uint32_t gi = wave_incl_scan32(gt), ei = wave_incl_scan32(eq);
      if (lane < C) {
        sh_cbase[0][lane] = gi - gt;
        sh_cbase[1][lane] = ei - eq;
      }
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const uint32_t mine = counts(c);
      const uint32_t excl = wave_incl_scan32(mine) - mine + sh_wbase[wave][c];
      uint32_t gt_before = sh_cbase[0][c] + (excl >> 16);
      uint32_t eq_before = sh_cbase[1][c] + (excl & 0xffffu);
      if (c * NT < vld_n) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int32_t p = 4 * (c * NT + t) + q;
          if (keys[c][q] > cut) {
            const uint32_t o = gt_before + min(eq_before, take_eq);
            if (o < static_cast<uint32_t>(k)) out[o] = p;
            ++gt_before;
          } else if (keys[c][q] == cut) {
            if (eq_before < take_eq) {
              const uint32_t o = gt_before + eq_before;
              if (o < static_cast<uint32_t>(k)) out[o] = p;
            }
            ++eq_before;
          }
        }
      }
    }
  }
  if (nan_out) write_block_total<NT>(nan, sh_scan, nan_out + blockIdx.x);
}

__global__ __launch_bounds__(kSelThreads, 1)
void order_stat_kernel(const float* __restrict__ score, const int32_t* __restrict__ n_dev, int n_max,
                       int rank, float* __restrict__ tau_out, int32_t* __restrict__ nan_out) {
  __shared__ uint32_t hist[kCopies * kBins];
  __shared__ uint64_t sh_scan[2 * kSelWaves + 8];
  __shared__ uint32_t sh_cut[2];
  int n = n_dev ? *n_dev : n_max;
  if (n > n_max) n = n_max;
  if (n < 0) n = 0;
  if (nan_out) {
    uint32_t nan = 0u;
    for (int i = threadIdx.x; i < n; i += kSelThreads) nan += score_key(score[i]) == 0u;
    write_block_total<kSelThreads>(nan, sh_scan, nan_out);
  }
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
                      int patience, uint8_t* __restrict__ counters, int n_counters, int32_t* __restrict__ out,
                      int32_t* __restrict__ n_out, int32_t* __restrict__ nan_out) {
  __shared__ uint64_t sh_scan[2 * kSelWaves + 8];
  int n = n_dev ? *n_dev : n_max;
  if (n > n_max) n = n_max;
  if (n < 0) n = 0;
  const float tau = *tau_p;
  constexpr int E = 16;  // consecutive rows per thread per chunk; all loads issued before use
  uint32_t before = 0u, nan = 0u;
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
    for (int e = 0; e < E; ++e) {
      nan += (i0 + e < n && score_key(sc[e]) == 0u) ? 1u : 0u;
      if (p[e] >= n_counters) p[e] = -1;  // position outside the counters: the row is dropped
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
  if (nan_out) write_block_total<kSelThreads>(nan, sh_scan, nan_out);
}

}  // namespace

namespace {

// ---------------------------------------------------------------------------
// Batched rows: one wave per row, no workgroup barrier anywhere.  Lane l holds
// the keys of positions 256*j + 4*l + e (e < 4, j < J) in registers (one
// 16-byte load each).  Rows of more than 2048 scores first try the bracket
// above (wave_topk_bracket); the rest, and rows whose bracket misses, take the
// digit passes over every key described here.  The bits every key shares are settled from the wave's
// smallest and largest key; digits of up to 11 bits follow, counted into the
// wave's own 2048-bin LDS histogram.  The search stops as soon as the bin
// holding the cut is taken whole (its count equals the keys still wanted), and
// the emit then keeps every key >= that bin's lowest key: per 256-position
// chunk, four compare masks and the set bits of the lanes below (mbcnt) give
// each kept position its output slot.  Only a cut inside a run of equal keys
// takes the slower emit, which ranks the equal keys with wave scans.
// Full: the row fills all J chunks (n == 256 * J), so no position tests.
// Rows are n % 4 == 0 scores, 16-byte aligned.
// ---------------------------------------------------------------------------
constexpr int kWaveRowsPerBlock = 1;  // one row per workgroup: a slow row holds up no other row's slot

__device__ __forceinline__ void wave_lds_fence() { __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront"); }

// LDS word of histogram bin b in the one-wave kernel: bins are permuted
// within each group of 32 so that the scan, where lane l reads bins 32l + i
// for i = 0..31, touches 32 banks per read instead of 2.
__device__ __forceinline__ uint32_t wave_bin_word(uint32_t b) { return b ^ ((b >> 5) & 31u); }

// Number of lanes below this one whose bit is set in m.
__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u));
}

// ---------------------------------------------------------------------------
// Bracketed one-wave top-k (rows of more than 2048 scores).  The digit passes
// over every key are most of the one-wave kernel's instructions (a bin
// address, a prefix test and an LDS atomic per key and pass); here they run
// over a few hundred keys instead:
//  1. A fixed sample of 16 keys per lane (chunks spread over the row) is
//     counted into the histogram of the digit right below the sample's common
//     key prefix.  The sample ranks r - d and r + d around the cut's expected
//     rank r = k m / n (m sampled keys, d = three binomial standard deviations
//     plus two) name two bins whose outer edges bound a score interval
//     [lo, hi] that holds the cut unless the sample misleads.
//  2. One compare pass over the row counts the scores above hi and stores the
//     scores inside [lo, hi] in lane-private LDS slots.
//  3. If fewer than k scores lie above hi, at least k lie at or above lo and
//     every candidate found a slot, the cut is the (k - above)-th largest
//     candidate, found by the usual digit passes over the candidates alone.
//  4. The emit compares every score of the row with the cut.
// Every decision is a float compare, which ranks -0 and +0 as equal and NaN
// below every number, exactly as the keys do.  A row whose bracket misses
// returns false and takes the digit passes over all its keys: the result is
// the same either way, only the time differs.
// ---------------------------------------------------------------------------
constexpr int kCandRows = 32;  // candidate slots per lane

// Bins holding the keys of ranks R[t] (1-based, counted from the largest) in
// the wave's histogram of nb bins: bin[t], the rank within that bin
// (rank_in[t]) and the bin's count (cnt[t]); ok[t] is false when R[t] lies
// outside 1..total.  tot = number of keys counted.  Two levels: the lane whose
// 32 bins hold the rank (a scan of the lane totals), then the bin among those
// 32 (one bin per lane, a second scan).
template <int NTGT>
__device__ __forceinline__ void wave_find_bins(const uint32_t* h, const uint32_t (&R)[NTGT], int lane,
                                               uint32_t& tot, uint32_t (&bin)[NTGT], uint32_t (&rank_in)[NTGT],
                                               uint32_t (&cnt)[NTGT], bool (&ok)[NTGT]) {
  constexpr int kBPL = kBins / kWave;
  const uint32_t b0 = static_cast<uint32_t>(lane) * kBPL;
  uint32_t mine = 0u;
#pragma unroll
  for (int b = 0; b < kBPL; ++b) mine += h[wave_bin_word(b0 + b)];  // unused bins stay zero
  const uint32_t incl = wave_incl_scan32(mine);
  tot = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(incl), kWave - 1));
  const uint32_t above_lane = tot - incl;  // keys in the bins of the lanes above
  uint32_t src[NTGT], rin[NTGT], c[NTGT];
#pragma unroll
  for (int t = 0; t < NTGT; ++t) {
    const uint64_t who = __ballot(above_lane < R[t] && R[t] <= above_lane + mine);
    ok[t] = who != 0ull;
    src[t] = ok[t] ? static_cast<uint32_t>(__builtin_ctzll(who)) : 0u;
    rin[t] = R[t] - static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(above_lane), static_cast<int>(src[t])));
    c[t] = lane < kBPL ? h[wave_bin_word(src[t] * kBPL + static_cast<uint32_t>(lane))] : 0u;
  }
#pragma unroll
  for (int t = 0; t < NTGT; ++t) {
    const uint32_t ci = wave_incl_scan32(c[t]);
    const uint32_t ltot = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(ci), kBPL - 1));
    const uint32_t above = ltot - ci;  // keys in this lane's higher bins
    const uint64_t who = __ballot(lane < kBPL && above < rin[t] && rin[t] <= above + c[t]);
    const int bl = who != 0ull ? static_cast<int>(__builtin_ctzll(who)) : 0;
    ok[t] = ok[t] && who != 0ull;
    bin[t] = src[t] * kBPL + static_cast<uint32_t>(bl);
    rank_in[t] = rin[t] - static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(above), bl));
    cnt[t] = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(c[t]), bl));
  }
}

__device__ __forceinline__ uint32_t wave_sum32(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(wave_incl_scan32(v)), kWave - 1));
}

__device__ __forceinline__ uint32_t wave_max32(uint32_t v) {
  v = wave_incl_scan_op(v, 0u, [](uint32_t a, uint32_t b) { return max(a, b); });
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), kWave - 1));
}

__device__ __forceinline__ uint32_t wave_min32(uint32_t v) {
  v = wave_incl_scan_op(v, 0xffffffffu, [](uint32_t a, uint32_t b) { return min(a, b); });
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), kWave - 1));
}

// raw[j][e]: the bits of the score at position 256 j + 4 lane + e.  Returns
// false (nothing written) when the bracket misses; true once the row's k
// outputs are written.  Needs 0 < k < n and J >= 16.
template <int J, bool Full>
__device__ __forceinline__ bool wave_topk_bracket(const uint32_t (&raw)[J][4], int lane, int n, int k,
                                                  uint32_t* h, uint32_t* cand, int32_t* __restrict__ out) {
  static_assert(J >= 16 && J % 16 == 0, "the sample takes one key of every J/16-th chunk");
  const int n4 = n >> 2;
  auto valid = [&](int j) { return Full || j * kWave + lane < n4; };
  constexpr int kS = 16;  // sampled keys per lane: key t & 3 of chunk t * J / 16

  // 1. the bracket from the sample
  uint32_t sk[kS];
  uint32_t smin = 0xffffffffu, smax = 0u, mine = 0u;
#pragma unroll
  for (int t = 0; t < kS; ++t) {
    sk[t] = score_key(__uint_as_float(raw[t * (J / 16)][t & 3]));
    if (valid(t * (J / 16))) {
      smin = min(smin, sk[t]);
      smax = max(smax, sk[t]);
      ++mine;
    }
  }
  smin = wave_min32(smin);
  smax = wave_max32(smax);
  const uint32_t m = wave_sum32(mine);
  if (m == 0u) return false;
  const int common = smin == smax ? 32 : __clz(smin ^ smax);
  const uint32_t sprefix = smin & static_cast<uint32_t>(0xffffffff00000000ull >> common);
  const int rem = 32 - common;
  const int wd = rem < 11 ? rem : 11;
  const int sh = rem - wd;
  const uint32_t dm = (1u << wd) - 1u;
#pragma unroll
  for (int b = 0; b < kBins / kWave / 4; ++b) reinterpret_cast<u32x4*>(h)[b * kWave + lane] = u32x4{0u, 0u, 0u, 0u};
  wave_lds_fence();
#pragma unroll
  for (int t = 0; t < kS; ++t)
    atomicAdd(&h[wave_bin_word((sk[t] >> sh) & dm)], valid(t * (J / 16)) ? 1u : 0u);
  wave_lds_fence();
  const float p = static_cast<float>(k) / static_cast<float>(n);
  const float r = p * static_cast<float>(m);
  const float d = 3.0f * __builtin_sqrtf(static_cast<float>(m) * p * (1.0f - p)) + 2.0f;
  const float rh = __builtin_floorf(r - d), rl = __builtin_ceilf(r + d);
  const bool has_hi = rh >= 1.0f, has_lo = rl <= static_cast<float>(m);
  const uint32_t R[2] = {has_hi ? static_cast<uint32_t>(rh) : 1u, has_lo ? static_cast<uint32_t>(rl) : m};
  uint32_t stot, sbin[2], srank[2], scnt[2];
  bool sok[2];
  wave_find_bins<2>(h, R, lane, stot, sbin, srank, scnt, sok);
  float hi_f = __builtin_inff(), lo_f = -__builtin_inff();
  if (has_hi) {
    const uint32_t hk = sprefix | (sbin[0] << sh) | ((1u << sh) - 1u);  // top key of the bin
    if (!sok[0] || hk < 0x007fffffu) return false;  // the sample's upper ranks are NaN
    if (hk < 0xff800000u) hi_f = key_score(hk);
  }
  if (has_lo) {
    const uint32_t lk = sprefix | (sbin[1] << sh);  // bottom key of the bin
    if (!sok[1]) return false;
    if (lk > 0x007fffffu) lo_f = key_score(lk);
  }

  // 2. one compare pass: count above hi, store [lo, hi] in lane-private slots
  // (lane l's i-th candidate in word i * 64 + l).  Every key is stored at the
  // lane's next free slot and the slot advances only for candidates, so no
  // per-key select of the address; a lane whose slots may run out before a
  // chunk is clamped to the last four rows and flagged, and its row falls back.
  uint32_t above = 0u;
  const uint32_t base = static_cast<uint32_t>(lane) * 4u;
  const uint32_t last = base + static_cast<uint32_t>(kCandRows - 4) * kWave * 4u;
  uint32_t addr = base;  // byte offset of the next free slot
  bool ovf = false;
  char* cb = reinterpret_cast<char*>(cand);
#pragma unroll
  for (int jj = 0; jj < J; ++jj) {  // chunk order is free here; even chunks arrived first
    const int j = jj < J / 2 ? 2 * jj : 2 * (jj - J / 2) + 1;
    const bool vj = valid(j);
    ovf = ovf || addr > last;
    addr = min(addr, last);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float x = __uint_as_float(raw[j][e]);
      const bool a = vj && x > hi_f;
      const bool in = vj && x >= lo_f && !a;
      above += static_cast<uint32_t>(__popcll(__ballot(a)));
      *reinterpret_cast<uint32_t*>(cb + addr) = raw[j][e];
      addr += in ? static_cast<uint32_t>(kWave * 4) : 0u;
    }
    __builtin_amdgcn_sched_barrier(0);  // chunk by chunk: no compare results of later chunks held early
  }
  const uint32_t cnt = (addr - base) / static_cast<uint32_t>(kWave * 4);
  const uint32_t cmax = wave_max32(cnt);
  const uint32_t ctot = wave_sum32(cnt);
  if (__ballot(ovf) != 0ull || above >= static_cast<uint32_t>(k) || above + ctot < static_cast<uint32_t>(k))
    return false;

  // 3. the (k - above)-th largest candidate: digit passes below the bits that
  // every key in [lo, hi] shares
  wave_lds_fence();
  uint32_t kk = static_cast<uint32_t>(k) - above;
  const uint32_t klo = score_key(lo_f), khi = score_key(hi_f);
  const int common2 = klo == khi ? 32 : __clz(klo ^ khi);
  uint32_t pmask = static_cast<uint32_t>(0xffffffff00000000ull >> common2);
  uint32_t prefix = klo & pmask;
  int sh2 = 32 - common2;
  bool whole = sh2 == 0 && kk == ctot;
#pragma unroll 1
  while (sh2 > 0) {
    const int wd2 = sh2 < 11 ? sh2 : 11;
    sh2 -= wd2;
    const uint32_t dm2 = (1u << wd2) - 1u;
#pragma unroll
    for (int b = 0; b < kBins / kWave / 4; ++b) reinterpret_cast<u32x4*>(h)[b * kWave + lane] = u32x4{0u, 0u, 0u, 0u};
    wave_lds_fence();
#pragma unroll 4
    for (uint32_t t = 0; t < cmax; ++t) {
      const uint32_t key = score_key(__uint_as_float(cand[t * kWave + lane]));
      atomicAdd(&h[wave_bin_word((key >> sh2) & dm2)], (t < cnt && (key & pmask) == prefix) ? 1u : 0u);
    }
    wave_lds_fence();
    uint32_t ctot2, bin[1], rin[1], bc[1];
    bool bok[1];
    const uint32_t Rk[1] = {kk};
    wave_find_bins<1>(h, Rk, lane, ctot2, bin, rin, bc, bok);
    prefix |= bin[0] << sh2;
    pmask |= dm2 << sh2;
    kk = rin[0];
    if (kk == bc[0]) {
      whole = true;
      break;
    }
  }

  // 4. emit, ascending positions: chunk j, lane l's positions 256 j + 4 l + e
  // follow every kept position of the lanes below it
  if (whole) {
    // keep x >= t: everything above hi, and the candidates whose key is at
    // least the cut bin's lowest key
    const float t_f = fmaxf(lo_f, key_score(prefix));
    // stores through a buffer resource over the row's k outputs: the base
    // stays in scalar registers, a lane whose key is not kept stores to an
    // offset past the end (dropped by the hardware, so no branch per key), and
    // so is a store past the k-th slot (impossible while the counts hold)
    const __amdgpu_buffer_rsrc_t orsrc = __builtin_amdgcn_make_buffer_rsrc(
        out, static_cast<short>(0), k * static_cast<int>(sizeof(int32_t)), 0x00020000);
    uint32_t before = 0u;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      bool t[4];
      uint64_t mk[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        t[e] = valid(j) && __uint_as_float(raw[j][e]) >= t_f;
        mk[e] = __ballot(t[e]);
      }
      uint32_t ob = (before + lanes_below(mk[0]) + lanes_below(mk[1]) + lanes_below(mk[2]) + lanes_below(mk[3])) * 4u;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        __builtin_amdgcn_raw_buffer_store_b32(static_cast<uint32_t>(j * 4 * kWave + 4 * lane + e), orsrc,
                                              static_cast<int>(t[e] ? ob : 0x7ffffff0u), 0, 0);
        ob += t[e] ? 4u : 0u;
      }
      before += static_cast<uint32_t>(__popcll(mk[0]) + __popcll(mk[1]) + __popcll(mk[2]) + __popcll(mk[3]));
      __builtin_amdgcn_sched_barrier(0);
    }
    return true;
  }
  // the cut lies inside a run of scores equal to c: keep every greater score
  // and the first kk equal ones in position order
  const float c = key_score(prefix);
  const uint32_t take_eq = kk;
  uint32_t sel_before = 0u, eq_before = 0u;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    uint32_t gt_bits = 0u, eq_bits = 0u;
    if (valid(j)) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x = __uint_as_float(raw[j][e]);
        if (x > c) gt_bits |= 1u << e;
        else if (x == c) eq_bits |= 1u << e;
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
      if ((eq_bits >> e) & 1u) {
        take = eq_rank < take_eq;
        ++eq_rank;
      }
      if (take) {
        if (o < static_cast<uint32_t>(k)) out[o] = j * 4 * kWave + 4 * lane + e;
        ++o;
      }
    }
    const uint32_t tot_eq = tot & 0xffffu;
    sel_before += (tot >> 16) + (min(eq_before + tot_eq, take_eq) - min(eq_before, take_eq));
    eq_before += tot_eq;
  }
  return true;
}

template <int J, bool Full>
__global__ __launch_bounds__(kWaveRowsPerBlock * kWave, J >= 32 ? 2 : 3)
void topk_wave_kernel(const float* __restrict__ score, int rows, int n, int k, int32_t* __restrict__ idx,
                      int32_t* __restrict__ nan_out) {
  __shared__ uint32_t hist_all[kWaveRowsPerBlock * kBins];
  __shared__ uint32_t cand_all[J >= 16 ? kWaveRowsPerBlock * kCandRows * kWave : 1];
  const int lane = threadIdx.x & (kWave - 1);
  const int w = kWaveRowsPerBlock == 1 ? 0 : static_cast<int>(threadIdx.x) / kWave;  // uniform row base
  const int row = blockIdx.x * kWaveRowsPerBlock + w;
  if (row >= rows) return;  // the whole wave leaves; nothing below synchronises waves
  uint32_t* h = hist_all + w * kBins;
  const u32x4* r4 = reinterpret_cast<const u32x4*>(score + static_cast<size_t>(row) * n);
  int32_t* out = idx + static_cast<size_t>(row) * k;
  const int n4 = n >> 2;
  auto valid = [&](int j) { return Full || j * kWave + lane < n4; };
  uint32_t keys[J][4];
  // every load in flight before the first is used; even chunks first (with
  // 32 chunks the bracket's sample reads only those, so it waits for half the
  // loads)
#pragma unroll
  for (int jj = 0; jj < J; ++jj) {
    const int j = jj < J / 2 ? 2 * jj : 2 * (jj - J / 2) + 1;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (valid(j)) v = __builtin_nontemporal_load(r4 + j * kWave + lane);
#pragma unroll
    for (int e = 0; e < 4; ++e) keys[j][e] = v[e];
  }
  if (nan_out) {  // NaN scores: per-lane counts, then one wave sum
    uint32_t nan = 0u;
#pragma unroll
    for (int j = 0; j < J; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        nan += (valid(j) && (keys[j][e] & 0x7fffffffu) > 0x7f800000u) ? 1u : 0u;
        __builtin_amdgcn_sched_barrier(0);  // one key at a time: no 128 live compare results
      }
    nan = wave_incl_scan32(nan);
    if (lane == kWave - 1) nan_out[row] = static_cast<int32_t>(nan);
  }
  if constexpr (J >= 16) {
    if (k > 0 && k < n && wave_topk_bracket<J, Full>(keys, lane, n, k, h, cand_all + w * kCandRows * kWave, out))
      return;
  }
#pragma unroll
  for (int j = 0; j < J; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) keys[j][e] = score_key(__uint_as_float(keys[j][e]));

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
  // whole: every key of the bin that holds the cut is kept, so the kept keys
  // are exactly those >= prefix (the bin's lowest key).  With one key value
  // in the row, that is when all n are kept.
  bool whole = sh == 0 && kk == static_cast<uint32_t>(n);
#pragma unroll 1
  while (sh > 0) {
    const int wd = sh < 11 ? sh : 11;
    sh -= wd;
    const uint32_t dm = (1u << wd) - 1u;
#pragma unroll
    for (int b = 0; b < kBPL / 4; ++b) reinterpret_cast<u32x4*>(h)[b * kWave + lane] = u32x4{0u, 0u, 0u, 0u};
    wave_lds_fence();
    // Branch-free: every key adds 1 when it carries the prefix, else 0 (on the
    // first digit every key does); per-key branches would keep 128 compare
    // masks alive across the loop.
#pragma unroll
    for (int j = 0; j < J; ++j) {
      if (valid(j)) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          atomicAdd(&h[wave_bin_word((keys[j][e] >> sh) & dm)], (keys[j][e] & pmask) == prefix ? 1u : 0u);
      }
      __builtin_amdgcn_sched_barrier(0);  // no bin addresses of later chunks computed ahead
    }
    wave_lds_fence();
    const int nb = static_cast<int>(dm) + 1;
    const int b0 = lane * kBPL;
    uint32_t c[kBPL];
    uint32_t mine = 0u;
#pragma unroll
    for (int b = 0; b < kBPL; ++b) {
      c[b] = h[wave_bin_word(static_cast<uint32_t>(b0 + b))];  // bins >= nb stay zero
      mine += c[b];
    }
    const uint32_t incl = wave_incl_scan32(mine);
    const uint32_t tot = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(incl), kWave - 1));
    uint32_t upto = incl - mine;  // keys in bins below b0
    uint32_t found_bin = 0u, found_kk = 0u, found_cnt = 0u;
    bool found = false;
#pragma unroll
    for (int b = 0; b < kBPL; ++b) {
      upto += c[b];
      const uint32_t above = tot - upto;  // keys in bins above b0 + b
      if (b0 + b < nb && above < kk && kk <= above + c[b]) {
        found = true;
        found_bin = static_cast<uint32_t>(b0 + b);
        found_kk = kk - above;
        found_cnt = c[b];
      }
    }
    const uint64_t who = __ballot(found);
    const int src = static_cast<int>(__builtin_ctzll(who));
    const uint32_t bin = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(found_bin), src));
    const uint32_t cnt = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(found_cnt), src));
    kk = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(found_kk), src));
    prefix |= bin << sh;
    pmask |= dm << sh;
    if (kk == cnt) {
      whole = true;
      break;
    }
  }

  if (whole) {
    // Keep key >= prefix.  Chunk j: lane l's positions 256j + 4l + e follow
    // every kept position of the lanes below it.
    uint32_t before = 0u;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      bool t[4];
      uint64_t m[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        t[e] = valid(j) && keys[j][e] >= prefix;
        m[e] = __ballot(t[e]);
      }
      uint32_t o = before + lanes_below(m[0]) + lanes_below(m[1]) + lanes_below(m[2]) + lanes_below(m[3]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (t[e] && o < static_cast<uint32_t>(k)) out[o] = j * 4 * kWave + 4 * lane + e;
        o += t[e] ? 1u : 0u;
      }
      before += static_cast<uint32_t>(__popcll(m[0]) + __popcll(m[1]) + __popcll(m[2]) + __popcll(m[3]));
      __builtin_amdgcn_sched_barrier(0);  // chunk by chunk: no masks of later chunks held early
    }
    return;
  }

  // The cut falls inside a run of keys equal to `prefix`: keep every greater
  // key and the first kk equal ones in position order.  Chunk j covers
  // positions 256*j .. 256*j + 255, lane l its four positions 256*j + 4*l + e.
  const uint32_t cut = prefix, take_eq = kk;
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

// ---------------------------------------------------------------------------
// One long row over many workgroups (top-k of a single row longer than
// kMultiMin scores, with a workspace): the row is cut into slices of kMSlice
// consecutive scores, one workgroup each, and the radix select runs as a
// chain of short launches on the same stream:
//   minmax  - each slice's smallest and largest key and NaN count;
//   seed    - (one workgroup) the bits every key shares, the forced ends, the
//             kept count and NaN total;
//   hist    - each slice's histogram of the next digit of the keys that carry
//             the settled prefix (LDS, written out per slice);
//   scan    - (one workgroup) the slice histograms summed, the cut bin found;
//             hist/scan repeat up to three times and stop once the cut bin is
//             taken whole or every bit is settled;
//   count   - each slice's (greater, equal) counts against the cut;
//   emit    - each slice writes its kept positions after those of the slices
//             before it, ascending, ties to the lower position.
// The state between launches lives in the workspace; no global atomics and no
// grid-wide waits, so the result is deterministic.
// ---------------------------------------------------------------------------
constexpr int kMT = 256;                // threads per workgroup
constexpr int kMItems = 8;              // consecutive scores per thread
constexpr int kMSlice = kMT * kMItems;  // scores per workgroup
constexpr int kMultiMin = 32768;        // single rows longer than this take the chain

struct MultiWs {
  uint32_t* state;  // prefix, prefix mask, bits left, keys still wanted, taken whole
  uint32_t* wg;     // [G][4]: min key, max key, NaN count
  uint32_t* cnt;    // [G][2]: greater, equal
  uint32_t* hist;   // [G][kBins]
};

__device__ __forceinline__ void multi_keys(const float* __restrict__ r, int n, uint32_t (&key)[kMItems],
                                           int& valid) {
  const int i0 = static_cast<int>(blockIdx.x) * kMSlice + static_cast<int>(threadIdx.x) * kMItems;
  valid = min(kMItems, max(0, n - i0));
#pragma unroll
  for (int e = 0; e < kMItems; ++e) key[e] = (e < valid) ? score_key(r[i0 + e]) : 0u;
}

__global__ __launch_bounds__(kMT)
void topk_multi_minmax(const float* __restrict__ r, int n, MultiWs w) {
  __shared__ uint32_t sh[3 * (kMT / kWave)];
  uint32_t key[kMItems];
  int valid;
  multi_keys(r, n, key, valid);
  uint32_t kmin = 0xffffffffu, kmax = 0u, nan = 0u;
#pragma unroll
  for (int e = 0; e < kMItems; ++e) {
    if (e < valid) {
      kmin = min(kmin, key[e]);
      kmax = max(kmax, key[e]);
      nan += key[e] == 0u;
    }
  }
  kmin = wave_incl_scan_op(kmin, 0xffffffffu, [](uint32_t a, uint32_t b) { return min(a, b); });
  kmax = wave_incl_scan_op(kmax, 0u, [](uint32_t a, uint32_t b) { return max(a, b); });
  nan = wave_incl_scan32(nan);
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
  if (lane == kWave - 1) {
    sh[wid] = kmin;
    sh[kMT / kWave + wid] = kmax;
    sh[2 * (kMT / kWave) + wid] = nan;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t a = sh[0], b = sh[kMT / kWave], c = sh[2 * (kMT / kWave)];
#pragma unroll
    for (int i = 1; i < kMT / kWave; ++i) {
      a = min(a, sh[i]);
      b = max(b, sh[kMT / kWave + i]);
      c += sh[2 * (kMT / kWave) + i];
    }
    w.wg[4 * blockIdx.x + 0] = a;
    w.wg[4 * blockIdx.x + 1] = b;
    w.wg[4 * blockIdx.x + 2] = c;
  }
}

// row: the whole row (n_row scores); the middle n_mid = n_row - f - l take part.
__global__ __launch_bounds__(kMT)
void topk_multi_seed(const float* __restrict__ row, int n_row, int k_total, int f, int l, int G,
                     const int32_t* __restrict__ pos, int32_t* __restrict__ out, int32_t* __restrict__ n_out,
                     int32_t* __restrict__ nan_out, MultiWs w) {
  __shared__ uint64_t sh_scan[2 * (kMT / kWave) + 8];
  __shared__ uint32_t sh_mm[2 * (kMT / kWave)];
  emit_forced<kMT>(n_row, k_total, f, l, pos, 0, out);
  uint32_t kmin = 0xffffffffu, kmax = 0u;
  uint32_t nan = nan_out ? forced_nans<kMT>(row, n_row, f, l) : 0u;
  for (int g = threadIdx.x; g < G; g += kMT) {
    kmin = min(kmin, w.wg[4 * g + 0]);
    kmax = max(kmax, w.wg[4 * g + 1]);
    nan += w.wg[4 * g + 2];
  }
  kmin = wave_incl_scan_op(kmin, 0xffffffffu, [](uint32_t a, uint32_t b) { return min(a, b); });
  kmax = wave_incl_scan_op(kmax, 0u, [](uint32_t a, uint32_t b) { return max(a, b); });
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
  if (lane == kWave - 1) {
    sh_mm[wid] = kmin;
    sh_mm[kMT / kWave + wid] = kmax;
  }
  uint64_t tot;
  (void)block_excl_scan<kMT>(nan, sh_scan, tot);  // also orders the sh_mm writes before the reads below
  if (threadIdx.x == 0) {
#pragma unroll
    for (int i = 1; i < kMT / kWave; ++i) {
      sh_mm[0] = min(sh_mm[0], sh_mm[i]);
      sh_mm[kMT / kWave] = max(sh_mm[kMT / kWave], sh_mm[kMT / kWave + i]);
    }
    const uint32_t a = sh_mm[0], b = sh_mm[kMT / kWave];
    if (nan_out) *nan_out = static_cast<int32_t>(tot);
    if (n_out) *n_out = k_total;
    const int common = a == b ? 32 : __clz(a ^ b);
    const uint32_t pmask = static_cast<uint32_t>(0xffffffff00000000ull >> common);
    const uint32_t kk = static_cast<uint32_t>(k_total - f - l);
    const int n_mid = n_row - f - l;
    w.state[0] = a & pmask;
    w.state[1] = pmask;
    w.state[2] = static_cast<uint32_t>(32 - common);
    w.state[3] = kk;
    w.state[4] = (common == 32 && kk == static_cast<uint32_t>(n_mid)) ? 1u : 0u;
  }
}

__global__ __launch_bounds__(kMT)
void topk_multi_hist(const float* __restrict__ r, int n, MultiWs w) {
  __shared__ uint32_t h[kBins];
  const uint32_t prefix = w.state[0], pmask = w.state[1];
  const int sh = static_cast<int>(w.state[2]);
  if (w.state[4] != 0u || sh <= 0) return;  // settled: nothing to count
  const int wd = sh < 11 ? sh : 11;
  const int shift = sh - wd;
  const uint32_t dm = (1u << wd) - 1u;
  for (int b = threadIdx.x; b < kBins; b += kMT) h[b] = 0u;
  uint32_t key[kMItems];
  int valid;
  multi_keys(r, n, key, valid);
  __syncthreads();
#pragma unroll
  for (int e = 0; e < kMItems; ++e)
    if (e < valid && (key[e] & pmask) == prefix) atomicAdd(&h[(key[e] >> shift) & dm], 1u);
  __syncthreads();
  uint32_t* gh = w.hist + static_cast<size_t>(blockIdx.x) * kBins;
  for (int b = threadIdx.x; b < kBins; b += kMT) gh[b] = h[b];
}

constexpr int kScanT = 1024;  // one workgroup, two bins per thread

__global__ __launch_bounds__(kScanT)
void topk_multi_scan(int G, MultiWs w) {
  __shared__ uint64_t sh_scan[2 * (kScanT / kWave) + 8];
  const uint32_t prefix = w.state[0], pmask = w.state[1], kk = w.state[3];
  const int sh = static_cast<int>(w.state[2]);
  if (w.state[4] != 0u || sh <= 0) return;
  const int wd = sh < 11 ? sh : 11;
  const int shift = sh - wd;
  const uint32_t dm = (1u << wd) - 1u;
  const int nb = static_cast<int>(dm) + 1;
  const int b0 = 2 * static_cast<int>(threadIdx.x);
  // this thread's two bins summed over the slices, 16 slices' loads in flight
  // at a time (addresses clamped into the slices that exist)
  uint32_t c0 = 0u, c1 = 0u;
  constexpr int kBatch = 16;
  for (int g0 = 0; g0 < G; g0 += kBatch) {
    u32x2 v[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i)
      v[i] = *reinterpret_cast<const u32x2*>(w.hist + static_cast<size_t>(min(g0 + i, G - 1)) * kBins + b0);
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      c0 += g0 + i < G ? v[i][0] : 0u;
      c1 += g0 + i < G ? v[i][1] : 0u;
    }
  }
  uint64_t tot;
  const uint32_t below = static_cast<uint32_t>(block_excl_scan<kScanT>(c0 + c1, sh_scan, tot));
  // keys strictly above bin b = total - (keys in bins <= b); the cut bin b
  // satisfies above(b) < kk <= above(b) + count(b)
  const uint32_t c[2] = {c0, c1};
  uint32_t upto = below;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    upto += c[j];
    const uint32_t above = static_cast<uint32_t>(tot) - upto;
    if (b0 + j < nb && above < kk && kk <= above + c[j]) {
      w.state[0] = prefix | (static_cast<uint32_t>(b0 + j) << shift);
      w.state[1] = pmask | (dm << shift);
      w.state[2] = static_cast<uint32_t>(shift);
      w.state[3] = kk - above;
      w.state[4] = (kk - above == c[j]) ? 1u : 0u;
    }
  }
}

// Kept keys against the cut: whole -> every key >= cut; otherwise every key
// > cut and the first take_eq keys == cut in position order.
__device__ __forceinline__ void multi_flags(const uint32_t (&key)[kMItems], int valid, uint32_t cut, bool whole,
                                            uint32_t& gt_bits, uint32_t& eq_bits) {
  gt_bits = 0u;
  eq_bits = 0u;
#pragma unroll
  for (int e = 0; e < kMItems; ++e) {
    if (e < valid) {
      if (key[e] > cut || (whole && key[e] == cut)) gt_bits |= 1u << e;
      else if (key[e] == cut) eq_bits |= 1u << e;
    }
  }
}

__global__ __launch_bounds__(kMT)
void topk_multi_count(const float* __restrict__ r, int n, MultiWs w) {
  __shared__ uint64_t sh_scan[2 * (kMT / kWave) + 8];
  const uint32_t cut = w.state[0];
  const bool whole = w.state[4] != 0u;
  uint32_t key[kMItems];
  int valid;
  multi_keys(r, n, key, valid);
  uint32_t gt_bits, eq_bits;
  multi_flags(key, valid, cut, whole, gt_bits, eq_bits);
  uint64_t tot;
  (void)block_excl_scan<kMT>((static_cast<uint64_t>(__popc(gt_bits)) << 32) | __popc(eq_bits), sh_scan, tot);
  if (threadIdx.x == 0) {
    w.cnt[2 * blockIdx.x + 0] = static_cast<uint32_t>(tot >> 32);
    w.cnt[2 * blockIdx.x + 1] = static_cast<uint32_t>(tot & 0xffffffffu);
  }
}

// out: the outputs of the middle (the whole row's out + f); positions are
// f + i, or pos[f + i] with a position map.
__global__ __launch_bounds__(kMT)
void topk_multi_emit(const float* __restrict__ r, int n, int f, int k_mid, const int32_t* __restrict__ pos,
                     int32_t* __restrict__ out, MultiWs w) {
  __shared__ uint64_t sh_scan[2 * (kMT / kWave) + 8];
  const uint32_t cut = w.state[0], take_eq = w.state[3];
  const bool whole = w.state[4] != 0u;
  // (greater, equal) counts of the slices before this one
  uint64_t before = 0ull;
  for (int g = threadIdx.x; g < static_cast<int>(blockIdx.x); g += kMT)
    before += (static_cast<uint64_t>(w.cnt[2 * g]) << 32) | w.cnt[2 * g + 1];
  uint64_t tb;
  (void)block_excl_scan<kMT>(before, sh_scan, tb);
  const uint32_t gt_before = static_cast<uint32_t>(tb >> 32), eq_before = static_cast<uint32_t>(tb & 0xffffffffu);
  uint32_t key[kMItems];
  int valid;
  multi_keys(r, n, key, valid);
  uint32_t gt_bits, eq_bits;
  multi_flags(key, valid, cut, whole, gt_bits, eq_bits);
  uint64_t tot;
  const uint64_t excl =
      block_excl_scan<kMT>((static_cast<uint64_t>(__popc(gt_bits)) << 32) | __popc(eq_bits), sh_scan, tot);
  uint32_t eq_rank = eq_before + static_cast<uint32_t>(excl & 0xffffffffu);
  uint32_t o = gt_before + min(eq_before, take_eq) + static_cast<uint32_t>(excl >> 32) +
               (min(eq_rank, take_eq) - min(eq_before, take_eq));
  const int i0 = static_cast<int>(blockIdx.x) * kMSlice + static_cast<int>(threadIdx.x) * kMItems;
#pragma unroll
  for (int e = 0; e < kMItems; ++e) {
    bool take = (gt_bits >> e) & 1u;
    if ((eq_bits >> e) & 1u) {
      take = eq_rank < take_eq;
      ++eq_rank;
    }
    if (take) {
      if (o < static_cast<uint32_t>(k_mid)) out[o] = pos ? pos[f + i0 + e] : f + i0 + e;
      ++o;
    }
  }
}

// Threshold step over many workgroups (one row longer than kMultiMin rows,
// with a workspace): slice g's rows are updated (counters written, the same
// rule as threshold_kernel) and their survivors counted in one launch; the
// second launch writes each slice's survivors after those of the slices
// before it, re-reading the updated counters to tell them.  The slice counts
// live in the workspace (cnt[g] = survivors, NaN scores).
__device__ __forceinline__ int thr_rows(const int32_t* __restrict__ n_dev, int n_max) {
  int n = n_dev ? *n_dev : n_max;
  return max(0, min(n, n_max));
}

__global__ __launch_bounds__(kMT)
void threshold_multi_update(const float* __restrict__ score, const int32_t* __restrict__ pos,
                            const int32_t* __restrict__ n_dev, int n_max, const float* __restrict__ tau_p,
                            int patience, uint8_t* __restrict__ counters, int n_counters, MultiWs w) {
  __shared__ uint64_t sh_scan[2 * (kMT / kWave) + 8];
  const int n = thr_rows(n_dev, n_max);
  const int i0 = static_cast<int>(blockIdx.x) * kMSlice + static_cast<int>(threadIdx.x) * kMItems;
  if (static_cast<int>(blockIdx.x) * kMSlice >= n) return;  // the whole workgroup: no slice rows
  const float tau = *tau_p;
  int32_t p[kMItems];
  float sc[kMItems];
#pragma unroll
  for (int e = 0; e < kMItems; ++e) {
    const int i = min(i0 + e, n - 1);  // unconditional loads; rows past n are not used
    p[e] = pos ? pos[i] : i;
    sc[e] = score[i];
  }
  uint32_t kept = 0u, nan = 0u;
#pragma unroll
  for (int e = 0; e < kMItems; ++e) {
    if (i0 + e < n) {
      nan += score_key(sc[e]) == 0u;
      if (p[e] >= 0 && p[e] < n_counters) {  // positions outside the counters are dropped
        const uint32_t c = (sc[e] < tau) ? static_cast<uint32_t>(counters[p[e]]) + 1u : 0u;
        counters[p[e]] = static_cast<uint8_t>(c > 255u ? 255u : c);
        kept += c < static_cast<uint32_t>(patience);
      }
    }
  }
  uint64_t tot;
  (void)block_excl_scan<kMT>((static_cast<uint64_t>(kept) << 32) | nan, sh_scan, tot);
  if (threadIdx.x == 0) {
    w.cnt[2 * blockIdx.x + 0] = static_cast<uint32_t>(tot >> 32);
    w.cnt[2 * blockIdx.x + 1] = static_cast<uint32_t>(tot & 0xffffffffu);
  }
}

__global__ __launch_bounds__(kMT)
void threshold_multi_emit(const int32_t* __restrict__ pos, const int32_t* __restrict__ n_dev, int n_max,
                          int patience, const uint8_t* __restrict__ counters, int n_counters,
                          int32_t* __restrict__ out, int32_t* __restrict__ n_out, int32_t* __restrict__ nan_out,
                          int G, MultiWs w) {
  __shared__ uint64_t sh_scan[2 * (kMT / kWave) + 8];
  const int n = thr_rows(n_dev, n_max);
  const int g_used = (n + kMSlice - 1) / kMSlice;  // slices that hold rows (and wrote their counts)
  const int g = static_cast<int>(blockIdx.x);
  // survivors of the slices before this one (slice 0 also totals every slice)
  uint64_t before = 0ull, all = 0ull;
  for (int j = threadIdx.x; j < g_used; j += kMT) {
    const uint64_t v = (static_cast<uint64_t>(w.cnt[2 * j]) << 32) | w.cnt[2 * j + 1];
    if (j < g) before += v;
    all += v;
  }
  uint64_t tb, ta;
  (void)block_excl_scan<kMT>(before, sh_scan, tb);
  if (g == 0) {
    (void)block_excl_scan<kMT>(all, sh_scan, ta);
    if (threadIdx.x == 0) {
      *n_out = static_cast<int32_t>(ta >> 32);
      if (nan_out) *nan_out = static_cast<int32_t>(ta & 0xffffffffu);
    }
  }
  if (g >= g_used) return;
  const int i0 = g * kMSlice + static_cast<int>(threadIdx.x) * kMItems;
  uint32_t keep_bits = 0u;
  int32_t p[kMItems];
#pragma unroll
  for (int e = 0; e < kMItems; ++e) {
    const int i = min(i0 + e, n - 1);
    p[e] = pos ? pos[i] : i;
  }
#pragma unroll
  for (int e = 0; e < kMItems; ++e)
    if (i0 + e < n && p[e] >= 0 && p[e] < n_counters && counters[p[e]] < static_cast<uint32_t>(patience))
      keep_bits |= 1u << e;
  uint64_t tot;
  const uint32_t o0 = static_cast<uint32_t>(tb >> 32) +
                      static_cast<uint32_t>(block_excl_scan<kMT>(__popc(keep_bits), sh_scan, tot));
  uint32_t o = o0;
#pragma unroll
  for (int e = 0; e < kMItems; ++e)
    if (keep_bits & (1u << e)) {
      if (o < static_cast<uint32_t>(n_max)) out[o] = p[e];  // never beyond the capacity
      ++o;
    }
}

MultiWs multi_ws_layout(void* base, int G) {
  auto a256 = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
  unsigned char* p = static_cast<unsigned char*>(base);
  MultiWs w;
  w.state = reinterpret_cast<uint32_t*>(p);
  p += 256;
  w.wg = reinterpret_cast<uint32_t*>(p);
  p += a256(static_cast<size_t>(G) * 16);
  w.cnt = reinterpret_cast<uint32_t*>(p);
  p += a256(static_cast<size_t>(G) * 8);
  w.hist = reinterpret_cast<uint32_t*>(p);
  return w;
}

// n: the row length (ragged: the packed score count); n_longest: the longest
// row (picks the kernel); cu_n / cu_k: ragged layout or null; n_dev: device
// count of a single fixed row or null.
template <int NT>
void launch_topk_nt(const float* score, int rows, int n, int k, int f, int l, const int32_t* pos, int32_t* idx,
                    const int32_t* cu_n, const int32_t* cu_k, const int32_t* n_dev, int32_t* n_out,
                    int32_t* nan_out, hipStream_t stream, int n_longest = -1) {
  const int n_mid = cu_n ? n_longest : n - f - l;
  const dim3 g(rows), b(NT);
#define DASH_TOPK_ARGS score, n, k, f, l, pos, idx, cu_n, cu_k, n_dev, n_out, nan_out
  if (n_mid <= NT * 4)
    hipLaunchKernelGGL((topk_reg_kernel<NT, 4>), g, b, 0, stream, DASH_TOPK_ARGS);
  else if (n_mid <= NT * 8)
    hipLaunchKernelGGL((topk_reg_kernel<NT, 8>), g, b, 0, stream, DASH_TOPK_ARGS);
  else if (n_mid <= NT * 16)
    hipLaunchKernelGGL((topk_reg_kernel<NT, 16>), g, b, 0, stream, DASH_TOPK_ARGS);
  else if (n_mid <= NT * 32)
    hipLaunchKernelGGL((topk_reg_kernel<NT, 32>), g, b, 0, stream, DASH_TOPK_ARGS);
  else if (rows == 1)
    hipLaunchKernelGGL((topk_kernel<NT, true>), g, b, 0, stream, DASH_TOPK_ARGS);
  else
    hipLaunchKernelGGL((topk_kernel<NT, false>), g, b, 0, stream, DASH_TOPK_ARGS);
#undef DASH_TOPK_ARGS
}

}  // namespace

// Many rows of at most 8192 aligned scores without forced ends, a position
// map or a device count: one wave per row.  Otherwise one 1024-thread
// workgroup per row.  k == 0 still launches when a count is to be written.
hipError_t launch_topk(const float* score, int rows, int n, int k, int keep_first, int keep_last,
                       const int32_t* pos, const int32_t* n_dev, int32_t* idx, int32_t* n_out, int32_t* nan_out,
                       hipStream_t stream) {
  if (rows == 0 || (k == 0 && !n_out && !nan_out)) return hipSuccess;
  const bool wave_rows = rows >= kWaveRowsMin && !pos && !n_dev && keep_first == 0 && keep_last == 0 &&
                         n % 4 == 0 && n <= 8192 && (reinterpret_cast<uintptr_t>(score) & 15u) == 0;
  if (wave_rows) {
    const dim3 grid((rows + kWaveRowsPerBlock - 1) / kWaveRowsPerBlock), block(kWaveRowsPerBlock * kWave);
#define DASH_WAVE_TOPK(J_)                                                                                 \
  do {                                                                                                     \
    if (n == 256 * (J_))                                                                                   \
      hipLaunchKernelGGL((topk_wave_kernel<J_, true>), grid, block, 0, stream, score, rows, n, k, idx, nan_out); \
    else                                                                                                   \
      hipLaunchKernelGGL((topk_wave_kernel<J_, false>), grid, block, 0, stream, score, rows, n, k, idx, nan_out); \
  } while (0)
    if (n <= 1024)
      DASH_WAVE_TOPK(4);
    else if (n <= 2048)
      DASH_WAVE_TOPK(8);
    else if (n <= 4096)
      DASH_WAVE_TOPK(16);
    else
      DASH_WAVE_TOPK(32);
#undef DASH_WAVE_TOPK
  } else if (rows >= 2 && !pos && !n_dev && !n_out && keep_first == 0 && keep_last == 0 && n % 4 == 0 &&
             n > kSelThreads * 32 && n <= kSelThreads * 64 && (reinterpret_cast<uintptr_t>(score) & 15u) == 0) {
    hipLaunchKernelGGL((topk_strided_kernel<kSelThreads, 16>), dim3(rows), dim3(kSelThreads), 0, stream, score, n, k,
                       idx, nan_out);
  } else {
    launch_topk_nt<kSelThreads>(score, rows, n, k, keep_first, keep_last, pos, idx, nullptr, nullptr, n_dev, n_out,
                                nan_out, stream);
  }
  return hipGetLastError();
}

size_t topk_multi_ws_bytes(int n_row, int keep_first, int keep_last) {
  const int n_mid = n_row - keep_first - keep_last;
  if (n_mid <= kMultiMin) return 0;
  const size_t G = static_cast<size_t>((n_mid + kMSlice - 1) / kMSlice);
  auto a256 = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
  return 256 + a256(G * 16) + a256(G * 8) + a256(G * kBins * 4);
}

hipError_t launch_topk_multi(const float* score, int n_row, int k_total, int keep_first, int keep_last,
                             const int32_t* pos, int32_t* idx, int32_t* n_out, int32_t* nan_out, void* scratch,
                             hipStream_t stream) {
  const int f = keep_first, l = keep_last;
  const int n_mid = n_row - f - l, k_mid = k_total - f - l;
  if (n_mid <= kMultiMin || k_mid <= 0 || !scratch) return hipErrorInvalidValue;
  const int G = (n_mid + kMSlice - 1) / kMSlice;
  const MultiWs w = multi_ws_layout(scratch, G);
  const float* r = score + f;
  hipLaunchKernelGGL(topk_multi_minmax, dim3(G), dim3(kMT), 0, stream, r, n_mid, w);
  hipLaunchKernelGGL(topk_multi_seed, dim3(1), dim3(kMT), 0, stream, score, n_row, k_total, f, l, G, pos, idx, n_out,
                     nan_out, w);
  for (int pass = 0; pass < 3; ++pass) {  // 32 key bits: at most 11 + 11 + 10
    hipLaunchKernelGGL(topk_multi_hist, dim3(G), dim3(kMT), 0, stream, r, n_mid, w);
    hipLaunchKernelGGL(topk_multi_scan, dim3(1), dim3(kScanT), 0, stream, G, w);
  }
  hipLaunchKernelGGL(topk_multi_count, dim3(G), dim3(kMT), 0, stream, r, n_mid, w);
  hipLaunchKernelGGL(topk_multi_emit, dim3(G), dim3(kMT), 0, stream, r, n_mid, f, k_mid, pos, idx + f, w);
  return hipGetLastError();
}

hipError_t launch_topk_ragged(const float* score, int n_total, int B, const int32_t* cu_n, const int32_t* cu_k,
                              int max_n, int k_cap, int keep_first, int keep_last, int32_t* idx, hipStream_t stream) {
  if (B == 0 || max_n == 0 || k_cap == 0 || n_total == 0) return hipSuccess;
  launch_topk_nt<kSelThreads>(score, B, n_total, k_cap, keep_first, keep_last, nullptr, idx, cu_n, cu_k, nullptr,
                              nullptr, nullptr, stream, max_n);
  return hipGetLastError();
}

hipError_t launch_order_stat(const float* score, const int32_t* n_dev, int n_max, int rank, float* tau_out,
                             int32_t* nan_out, hipStream_t stream) {
  hipLaunchKernelGGL(order_stat_kernel, dim3(1), dim3(kSelThreads), 0, stream, score, n_dev, n_max, rank,
                     tau_out, nan_out);
  return hipGetLastError();
}

hipError_t launch_threshold_multi(const float* score, const int32_t* pos, const int32_t* n_dev, int n_max,
                                  const float* tau, int patience, uint8_t* counters, int n_counters, int32_t* out,
                                  int32_t* n_out, int32_t* nan_out, void* scratch, hipStream_t stream) {
  if (n_max <= kMultiMin || !scratch) return hipErrorInvalidValue;
  const int G = (n_max + kMSlice - 1) / kMSlice;
  const MultiWs w = multi_ws_layout(scratch, G);
  hipLaunchKernelGGL(threshold_multi_update, dim3(G), dim3(kMT), 0, stream, score, pos, n_dev, n_max, tau, patience,
                     counters, n_counters, w);
  hipLaunchKernelGGL(threshold_multi_emit, dim3(G), dim3(kMT), 0, stream, pos, n_dev, n_max, patience, counters,
                     n_counters, out, n_out, nan_out, G, w);
  return hipGetLastError();
}

hipError_t launch_threshold(const float* score, const int32_t* pos, const int32_t* n_dev, int n_max,
                            const float* tau, int patience, uint8_t* counters, int n_counters, int32_t* out,
                            int32_t* n_out, int32_t* nan_out, hipStream_t stream) {
  hipLaunchKernelGGL(threshold_kernel, dim3(1), dim3(kSelThreads), 0, stream, score, pos, n_dev, n_max, tau,
                     patience, counters, n_counters, out, n_out, nan_out);
  return hipGetLastError();
}

}  // namespace dash
