// Compaction of active rows: Xa[r] = X[idx[r]] — the gather of the selected
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

__global__ __launch_bounds__(kCompactThreads)
void compact_kernel(const int32_t* __restrict__ idx, const int32_t* __restrict__ n_dev, int n_max,
                    const u32x4* __restrict__ X, int S, uint32_t cpr, u32x4* __restrict__ Xa) {
  int n = n_dev ? *n_dev : n_max;
  if (n > n_max) n = n_max;
  // The host guarantees n_max * cpr < 2^31, so 32-bit indexing is exact.
  const uint32_t total = static_cast<uint32_t>(n < 0 ? 0 : n) * cpr;
  const uint32_t base = blockIdx.x * (kCompactItems * kCompactThreads) + threadIdx.x;
  u32x4 v[kCompactItems];
  uint32_t dst[kCompactItems];
  bool ok[kCompactItems];
#pragma unroll
  for (int it = 0; it < kCompactItems; ++it) {
    const uint32_t e = base + static_cast<uint32_t>(it) * kCompactThreads;
    ok[it] = false;
    if (e < total) {
      const uint32_t r = e / cpr;
      const uint32_t c = e - r * cpr;
      const int32_t src = idx[r];
      if (src >= 0 && src < S) {
        v[it] = __builtin_nontemporal_load(X + static_cast<uint64_t>(src) * cpr + c);
        dst[it] = e;
        ok[it] = true;
      }
    }
  }
#pragma unroll
  for (int it = 0; it < kCompactItems; ++it)
    if (ok[it]) Xa[dst[it]] = v[it];
}

}  // namespace

hipError_t launch_compact(const int32_t* idx, const int32_t* n_dev, int n_max, const void* X, int S,
                          size_t row_bytes, void* Xa, hipStream_t stream) {
  if (n_max <= 0) return hipSuccess;
  const uint32_t cpr = static_cast<uint32_t>(row_bytes / 16);
  const uint64_t total = static_cast<uint64_t>(n_max) * cpr;
  const uint64_t per_block = static_cast<uint64_t>(kCompactThreads) * kCompactItems;
  const uint64_t blocks = (total + per_block - 1) / per_block;
  if (blocks == 0) return hipSuccess;
  if (total >= 0x80000000ull) return hipErrorInvalidValue;
  hipLaunchKernelGGL(compact_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kCompactThreads), 0, stream, idx,
                     n_dev, n_max, static_cast<const u32x4*>(X), S, cpr, static_cast<u32x4*>(Xa));
  return hipGetLastError();
}

}  // namespace dash
