// Δattn score from a given U: score[t] = ||U_t||_2 — the token's update from
// the attention sublayer, CSDN explainer "DASH：基于注意力增量的Transformer令牌
// 压缩，实现长序列推理高效加速", §2.1 (definition) and §2.2 (only U is needed, so
// the score works with any attention kernel that produces U).
//
// HBM-bound row reduction: one wave per row, each lane reading 16-byte chunks
// of the row (consecutive lanes, consecutive chunks), fp32 sums of squares,
// a fixed-order wave reduction, one sqrt.  The grid is sized from the row
// capacity so a device-resident row count needs no host round trip.
#include "dash_common.h"
#include "dash_kernels.h"

namespace dash {

namespace {

constexpr int kScoreWaves = 4;  // rows per workgroup

__device__ __forceinline__ float sq_sum(const u32x4& v, int dtype) {
  float s = 0.f;
  if (dtype == 1) {  // eight bf16
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float lo = __uint_as_float(v[w] << 16);
      const float hi = __uint_as_float(v[w] & 0xffff0000u);
      s += lo * lo;
      s += hi * hi;
    }
  } else {  // four fp32
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float x = __uint_as_float(v[w]);
      s += x * x;
    }
  }
  return s;
}

template <int DT>
__global__ __launch_bounds__(kScoreWaves * kWave)
void row_norm_kernel(const u32x4* __restrict__ U, const int32_t* __restrict__ n_dev, int n_max, int chunks,
                     float* __restrict__ score) {
  int n = n_dev ? *n_dev : n_max;
  if (n > n_max) n = n_max;
  const int row = blockIdx.x * kScoreWaves + static_cast<int>(threadIdx.x / kWave);
  if (row >= n) return;
  const int lane = threadIdx.x & (kWave - 1);
  const u32x4* r = U + static_cast<size_t>(row) * chunks;
  constexpr int kU = 4;  // loads in flight per lane
  float s = 0.f;
  int c = lane;
  for (; c + (kU - 1) * kWave < chunks; c += kU * kWave) {
    u32x4 v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) v[u] = __builtin_nontemporal_load(r + c + u * kWave);
#pragma unroll
    for (int u = 0; u < kU; ++u) s += sq_sum(v[u], DT);
  }
  for (; c < chunks; c += kWave) s += sq_sum(__builtin_nontemporal_load(r + c), DT);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off, kWave);
  if (lane == 0) score[row] = sqrtf(s);
}

}  // namespace

hipError_t launch_row_norm(int dtype, const void* U, const int32_t* n_dev, int n_max, int hidden, float* score,
                           hipStream_t stream) {
  if (n_max <= 0) return hipSuccess;
  const int esz = dtype == 1 ? 2 : 4;
  const int chunks = hidden * esz / 16;
  const dim3 grid((n_max + kScoreWaves - 1) / kScoreWaves);
  if (dtype == 1)
    hipLaunchKernelGGL(row_norm_kernel<1>, grid, dim3(kScoreWaves * kWave), 0, stream,
                       static_cast<const u32x4*>(U), n_dev, n_max, chunks, score);
  else
    hipLaunchKernelGGL(row_norm_kernel<0>, grid, dim3(kScoreWaves * kWave), 0, stream,
                       static_cast<const u32x4*>(U), n_dev, n_max, chunks, score);
  return hipGetLastError();
}

}  // namespace dash
