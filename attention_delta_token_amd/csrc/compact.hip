// Compaction of active rows: Xa[r] = X[idx[r]] (batched: Xa[b, r] = X[b, idx[b, r]]) — the gather of the selected
// tokens that later layers work on, from the CSDN explainer
// "DASH：基于注意力增量的Transformer令牌压缩，实现长序列推理高效加速", §3.1 step 4
// and §3.3 (gather by the active index set, avoiding needless copies).
//
// HBM-bound copy.  One wave moves one row: the row's source index is read
// once, every 16-byte chunk of the row (across the gathered tensors) is loaded
// before any is stored, consecutive lanes move consecutive chunks (coalesced
// for any row width), and the stores bypass the caches' write-allocate
// (nontemporal), which measured faster than a plain device-to-device copy of
// the same bytes after other work has left the caches dirty.  The grid is sized from the row capacity, so a
// device-resident row count needs no host round trip.
#include "dash_common.h"
#include "dash_kernels.h"

namespace dash {

namespace {

constexpr int kCompactThreads = 256;
constexpr int kCompactRows = kCompactThreads / 64;  // one row per wave

// Up to kMaxGather tensors gathered at the same rows.  A gathered row is the
// 16-byte chunks of row r of tensor 0, then of tensor 1, ...; lo[j] is the
// first chunk of tensor j within it, w[j] its chunks per row and cpr the
// gathered row length.  Unused slots have lo = cpr.
struct GatherSet {
  const u32x4* X[kMaxGather];
  u32x4* Xa[kMaxGather];
  int S[kMaxGather];
  uint32_t lo[kMaxGather];
  uint32_t w[kMaxGather];
  uint32_t cpr;
};

template <class T>
__device__ __forceinline__ T pick(const T (&a)[kMaxGather], int j) {
  // compile-time selects (no indexing of the argument block at run time)
  T v = a[0];
#pragma unroll
  for (int t = 1; t < kMaxGather; ++t)
    if (j == t) v = a[t];
  return v;
}

// U chunks per lane in flight: a row of up to 64 * U chunks moves in one batch.
template <int U>
__global__ __launch_bounds__(kCompactThreads)
void compact_kernel(const int32_t* __restrict__ idx, const int32_t* __restrict__ n_dev, int n_max, int per_sample,
                    GatherSet g) {
  int n = n_dev ? *n_dev : n_max;
  if (n > n_max) n = n_max;
  const int r = __builtin_amdgcn_readfirstlane(static_cast<int>(blockIdx.x) * kCompactRows + (threadIdx.x >> 6));
  if (r >= n) return;
  const int lane = threadIdx.x & 63;
  const int32_t src = idx[r];
  // batched: row r belongs to sample r / per_sample, whose source rows start at sample * S
  const uint64_t sample = per_sample > 0 ? static_cast<uint32_t>(r) / static_cast<uint32_t>(per_sample) : 0u;
  const uint32_t cpr = g.cpr;
  for (uint32_t c0 = 0; c0 < cpr; c0 += 64u * U) {
    u32x4 v[U];
    u32x4* dst[U];
#pragma unroll
    for (int i = 0; i < U; ++i) {
      const uint32_t c = c0 + static_cast<uint32_t>(lane + 64 * i);
      dst[i] = nullptr;
      if (c < cpr) {
        int j = 0;
#pragma unroll
        for (int t = 1; t < kMaxGather; ++t)
          if (c >= g.lo[t]) j = t;
        const int Sj = pick(g.S, j);
        if (src >= 0 && src < Sj) {
          const uint32_t cj = c - pick(g.lo, j);
          const uint32_t w = pick(g.w, j);
          v[i] = __builtin_nontemporal_load(pick(g.X, j) + (sample * Sj + static_cast<uint64_t>(src)) * w + cj);
          dst[i] = pick(g.Xa, j) + static_cast<uint64_t>(r) * w + cj;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < U; ++i)
      if (dst[i]) __builtin_nontemporal_store(v[i], dst[i]);
  }
}

// Rows of at most 64 * U chunks per tensor (U = 1: 1 KiB, 2: 2 KiB), e.g. the
// K and V rows of a kv-head group, C tensors: each tensor's source row
// address is scalar and a chunk costs one address add.  Every load is issued
// unconditionally (a lane past the row's width re-reads the row's last chunk;
// a source index outside the tensor reads the destination row instead), so
// all of a row's loads are in flight before the first store; only the stores
// are conditional.
template <int U, int C>
__global__ __launch_bounds__(kCompactThreads)
void compact_rows_kernel(const int32_t* __restrict__ idx, const int32_t* __restrict__ n_dev, int n_max,
                         int per_sample, GatherSet g) {
  int n = n_max;
  if (n_dev) n = min(*n_dev, n_max);
  const int r = __builtin_amdgcn_readfirstlane(static_cast<int>(blockIdx.x) * kCompactRows + (threadIdx.x >> 6));
  if (r >= n) return;
  const int lane = threadIdx.x & 63;
  const int32_t src = idx[r];
  uint64_t sample = 0;
  if (per_sample > 0) sample = static_cast<uint32_t>(r) / static_cast<uint32_t>(per_sample);
  u32x4 v[C][U];
  bool ok[C];
#pragma unroll
  for (int j = 0; j < C; ++j) {
    // branch-free selection of the row address, so every descriptor field is
    // loaded up front instead of behind a branch
    const uint32_t w = g.w[j];
    ok[j] = static_cast<uint32_t>(src) < static_cast<uint32_t>(g.S[j]);
    const uint64_t s_off = (sample * static_cast<uint64_t>(static_cast<uint32_t>(g.S[j])) +
                            static_cast<uint64_t>(static_cast<uint32_t>(src))) * w;
    const uint64_t d_off = static_cast<uint64_t>(r) * w;
    const u32x4* row = ok[j] ? g.X[j] + s_off : g.Xa[j] + d_off;
#pragma unroll
    for (int u = 0; u < U; ++u)
      v[j][u] = __builtin_nontemporal_load(row + min(static_cast<uint32_t>(lane + 64 * u), w - 1u));
  }
#pragma unroll
  for (int j = 0; j < C; ++j) {
    const uint32_t w = g.w[j];
    if (ok[j]) {
      u32x4* row = g.Xa[j] + static_cast<uint64_t>(r) * w;
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (static_cast<uint32_t>(lane + 64 * u) < w) __builtin_nontemporal_store(v[j][u], row + lane + 64 * u);
    }
  }
}

}  // namespace

hipError_t launch_compact_many(const int32_t* idx, const int32_t* n_dev, int n_max, const GatherItem* items,
                               int count, hipStream_t stream, int per_sample) {
  if (n_max <= 0 || count <= 0) return hipSuccess;
  if (count > kMaxGather) return hipErrorInvalidValue;
  GatherSet g{};
  uint32_t acc = 0;
  for (int j = 0; j < count; ++j) {
    g.X[j] = static_cast<const u32x4*>(items[j].X);
    g.Xa[j] = static_cast<u32x4*>(items[j].Xa);
    g.S[j] = items[j].S;
    g.lo[j] = acc;
    g.w[j] = static_cast<uint32_t>(items[j].row_bytes / 16);
    acc += g.w[j];
  }
  for (int j = count; j < kMaxGather; ++j) {
    g.X[j] = g.X[0];
    g.Xa[j] = g.Xa[0];
    g.S[j] = 0;
    g.lo[j] = acc;
    g.w[j] = 1;
  }
  g.cpr = acc;
  const uint64_t total = static_cast<uint64_t>(n_max) * acc;
  if (total >= 0x80000000ull) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>((static_cast<uint64_t>(n_max) + kCompactRows - 1) / kCompactRows));
  uint32_t wmax = 0;
  for (int j = 0; j < count; ++j) wmax = g.w[j] > wmax ? g.w[j] : wmax;
  if (wmax <= 128) {  // rows of at most 2 KiB per tensor
#define DASH_ROWS(U_, C_) \
  hipLaunchKernelGGL((compact_rows_kernel<U_, C_>), grid, dim3(kCompactThreads), 0, stream, idx, n_dev, n_max, per_sample, g)
#define DASH_ROWS_C(U_)              \
  switch (count) {                   \
    case 1: DASH_ROWS(U_, 1); break; \
    case 2: DASH_ROWS(U_, 2); break; \
    case 3: DASH_ROWS(U_, 3); break; \
    default: DASH_ROWS(U_, 4); break; \
  }
    if (wmax <= 64) {
      DASH_ROWS_C(1)
    } else {
      DASH_ROWS_C(2)
    }
#undef DASH_ROWS_C
#undef DASH_ROWS
    return hipGetLastError();
  }
  const uint32_t need = (acc + 63) / 64;  // chunks per lane for one row
  if (need <= 1)
    hipLaunchKernelGGL(compact_kernel<1>, grid, dim3(kCompactThreads), 0, stream, idx, n_dev, n_max, per_sample, g);
  else if (need <= 2)
    hipLaunchKernelGGL(compact_kernel<2>, grid, dim3(kCompactThreads), 0, stream, idx, n_dev, n_max, per_sample, g);
  else if (need <= 4)
    hipLaunchKernelGGL(compact_kernel<4>, grid, dim3(kCompactThreads), 0, stream, idx, n_dev, n_max, per_sample, g);
  else if (need <= 8)
    hipLaunchKernelGGL(compact_kernel<8>, grid, dim3(kCompactThreads), 0, stream, idx, n_dev, n_max, per_sample, g);
  else if (need <= 12)
    hipLaunchKernelGGL(compact_kernel<12>, grid, dim3(kCompactThreads), 0, stream, idx, n_dev, n_max, per_sample, g);
  else
    hipLaunchKernelGGL(compact_kernel<16>, grid, dim3(kCompactThreads), 0, stream, idx, n_dev, n_max, per_sample, g);
  return hipGetLastError();
}

hipError_t launch_compact(const int32_t* idx, const int32_t* n_dev, int n_max, const void* X, int S,
                          size_t row_bytes, void* Xa, hipStream_t stream) {
  const GatherItem one{X, S, row_bytes, Xa};
  return launch_compact_many(idx, n_dev, n_max, &one, 1, stream, 0);
}

}  // namespace dash
