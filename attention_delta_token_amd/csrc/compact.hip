// Compaction of active rows: Xa[r] = X[idx[r]] (batched: Xa[b, r] = X[b, idx[b, r]]) — the gather of the selected
// tokens that later layers work on, from the CSDN explainer
// "DASH：基于注意力增量的Transformer令牌压缩，实现长序列推理高效加速", §3.1 step 4
// and §3.3 (gather by the active index set, avoiding needless copies).
//
// HBM-bound copy.  The (row, 16-byte chunk) space is flattened so that
// consecutive lanes move consecutive 16-byte chunks of one row (coalesced
// reads and writes for any row width), each thread moves several chunks with
// all loads issued before the stores, and the grid is sized from the row
// capacity so a device-resident row count needs no host round trip.
#include "dash_common.h"
#include "dash_kernels.h"

namespace dash {

namespace {

constexpr int kCompactThreads = 256;
constexpr int kCompactItems = 4;

// Up to kMaxGather tensors gathered at the same rows.  Row r of the flattened
// space holds the 16-byte chunks of row r of tensor 0, then of tensor 1, ...;
// lo[j] is the first chunk of tensor j within a flattened row, w[j] its chunks
// per row and cpr the flattened row length.  Unused slots have lo = cpr.
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

__global__ __launch_bounds__(kCompactThreads)
void compact_kernel(const int32_t* __restrict__ idx, const int32_t* __restrict__ n_dev, int n_max, int per_sample,
                    GatherSet g) {
  int n = n_dev ? *n_dev : n_max;
  if (n > n_max) n = n_max;
  const uint32_t cpr = g.cpr;
  // The host guarantees n_max * cpr < 2^31, so 32-bit indexing is exact.
  const uint32_t total = static_cast<uint32_t>(n < 0 ? 0 : n) * cpr;
  const uint32_t base = blockIdx.x * (kCompactItems * kCompactThreads) + threadIdx.x;
  u32x4 v[kCompactItems];
  u32x4* dst[kCompactItems];
#pragma unroll
  for (int it = 0; it < kCompactItems; ++it) {
    const uint32_t e = base + static_cast<uint32_t>(it) * kCompactThreads;
    dst[it] = nullptr;
    if (e < total) {
      const uint32_t r = e / cpr;
      const uint32_t c = e - r * cpr;
      int j = 0;
#pragma unroll
      for (int t = 1; t < kMaxGather; ++t)
        if (c >= g.lo[t]) j = t;
      const uint32_t cj = c - pick(g.lo, j);
      const uint32_t w = pick(g.w, j);
      const int32_t src = idx[r];
      const int Sj = pick(g.S, j);
      if (src >= 0 && src < Sj) {
        // batched: row r belongs to sample r / per_sample, whose rows start at sample * S
        const uint64_t base = per_sample > 0 ? static_cast<uint64_t>(r / static_cast<uint32_t>(per_sample)) * Sj : 0u;
        v[it] = __builtin_nontemporal_load(pick(g.X, j) + (base + static_cast<uint64_t>(src)) * w + cj);
        dst[it] = pick(g.Xa, j) + static_cast<uint64_t>(r) * w + cj;
      }
    }
  }
#pragma unroll
  for (int it = 0; it < kCompactItems; ++it)
    if (dst[it]) *dst[it] = v[it];
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
  const uint64_t per_block = static_cast<uint64_t>(kCompactThreads) * kCompactItems;
  const uint64_t blocks = (total + per_block - 1) / per_block;
  if (blocks == 0) return hipSuccess;
  if (total >= 0x80000000ull) return hipErrorInvalidValue;
  hipLaunchKernelGGL(compact_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kCompactThreads), 0, stream, idx,
                     n_dev, n_max, per_sample, g);
  return hipGetLastError();
}

hipError_t launch_compact(const int32_t* idx, const int32_t* n_dev, int n_max, const void* X, int S,
                          size_t row_bytes, void* Xa, hipStream_t stream) {
  const GatherItem one{X, S, row_bytes, Xa};
  return launch_compact_many(idx, n_dev, n_max, &one, 1, stream, 0);
}

}  // namespace dash
