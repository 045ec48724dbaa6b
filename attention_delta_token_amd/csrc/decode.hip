// Decode attention over a (pruned) KV cache — the step after a DASH prefill:
// the cache keeps only the active tokens, which shortens every later decode
// step (CSDN explainer "DASH：基于注意力增量的Transformer令牌压缩，实现长序列推理
// 高效加速", §3.1 step 5 and §5.1).
//
// Flash-decoding split over the keys: workgroup (chunk, kv-head, sample) reads
// its chunk of the cache once for all g q-heads x n_new new tokens of that
// kv-head (the rows of the group), keeps fp32 partials (row maximum, sum of
// exponentials, unnormalised output) in the workspace, and a second kernel
// merges the chunks in a fixed order.  The work per byte of cache is tiny, so
// the arithmetic is plain VALU over K/V tiles staged in LDS; what matters is
// that enough workgroups stream the cache at once.
#include "dash_common.h"
#include "dash_kernels.h"

namespace dash {

namespace {

constexpr int kDecThreads = 256;
constexpr int kDecTile = 64;     // keys per LDS tile
constexpr int kDecMaxRows = 32;     // g * n_new rows per workgroup
constexpr int kDecMaxChunks = 1024;  // key chunks per (sample, kv-head)

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(static_cast<uint32_t>(h) << 16); }

template <int D>
__global__ __launch_bounds__(kDecThreads)
void decode_chunk_kernel(const uint16_t* __restrict__ Qd, const uint16_t* __restrict__ Kc,
                         const uint16_t* __restrict__ Vc, const int32_t* __restrict__ n_kv_dev, int S_cap,
                         int n_new, int Hq, int Hkv, float c_log2, int chunk, int n_chunks,
                         float* __restrict__ part) {
  __shared__ float q_s[kDecMaxRows][D];
  __shared__ float o_s[kDecMaxRows][D];
  __shared__ float k_s[kDecTile][D + 1];
  __shared__ float v_s[kDecTile][D];
  __shared__ float p_s[kDecMaxRows][kDecTile];
  __shared__ float m_s[kDecMaxRows], l_s[kDecMaxRows], a_s[kDecMaxRows];
  const int c = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int g = Hq / Hkv;
  const int G = g * n_new;  // row r = token i * g + head offset jh
  const int tid = threadIdx.x;
  int n_kv = n_kv_dev[b];
  n_kv = max(0, min(n_kv, S_cap));
  const int k0 = c * chunk;
  const int k1 = min(k0 + chunk, n_kv);
  const int kv_ld = Hkv * D;
  const uint16_t* Kb = Kc + static_cast<int64_t>(b) * S_cap * kv_ld + static_cast<int64_t>(kvh) * D;
  const uint16_t* Vb = Vc + static_cast<int64_t>(b) * S_cap * kv_ld + static_cast<int64_t>(kvh) * D;
  for (int e = tid; e < G * D; e += kDecThreads) {
    const int r = e / D, d = e % D;
    const int i = r / g, jh = r % g;
    q_s[r][d] = bf16_to_f32(Qd[((static_cast<int64_t>(b) * n_new + i) * Hq + kvh * g + jh) * D + d]) * c_log2;
    o_s[r][d] = 0.f;
  }
  if (tid < G) {
    m_s[tid] = -__builtin_inff();
    l_s[tid] = 0.f;
  }
  __syncthreads();
  for (int t0 = k0; t0 < k1; t0 += kDecTile) {
    const int nt = min(kDecTile, k1 - t0);
    // 16-byte loads: 8 bf16 of one key row per thread and step
    for (int e = tid; e < kDecTile * (D / 8); e += kDecThreads) {
      const int j = e / (D / 8), d0 = (e % (D / 8)) * 8;
      u32x4 kv = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
      if (j < nt) {
        kv = *reinterpret_cast<const u32x4*>(Kb + static_cast<int64_t>(t0 + j) * kv_ld + d0);
        vv = *reinterpret_cast<const u32x4*>(Vb + static_cast<int64_t>(t0 + j) * kv_ld + d0);
      }
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        k_s[j][d0 + 2 * w] = __uint_as_float(kv[w] << 16);
        k_s[j][d0 + 2 * w + 1] = __uint_as_float(kv[w] & 0xffff0000u);
        v_s[j][d0 + 2 * w] = __uint_as_float(vv[w] << 16);
        v_s[j][d0 + 2 * w + 1] = __uint_as_float(vv[w] & 0xffff0000u);
      }
    }
    __syncthreads();
    // scores (exp2 units); a key is visible to token i iff its cache row <= n_kv - n_new + i
    for (int e = tid; e < G * kDecTile; e += kDecThreads) {
      const int r = e / kDecTile, j = e % kDecTile;
      const int qrow = n_kv - n_new + r / g;
      float sc = -__builtin_inff();
      if (j < nt && t0 + j <= qrow) {
        sc = 0.f;
#pragma unroll 8
        for (int d = 0; d < D; ++d) sc += q_s[r][d] * k_s[j][d];
      }
      p_s[r][j] = sc;
    }
    __syncthreads();
    // online softmax, one thread per row
    if (tid < G) {
      float mx = m_s[tid];
      for (int j = 0; j < nt; ++j) mx = fmaxf(mx, p_s[tid][j]);
      const float alpha = mx == -__builtin_inff() ? 1.f : __builtin_amdgcn_exp2f(m_s[tid] - mx);
      float sum = 0.f;
      for (int j = 0; j < kDecTile; ++j) {
        const float pj = (j < nt && mx != -__builtin_inff()) ? __builtin_amdgcn_exp2f(p_s[tid][j] - mx) : 0.f;
        p_s[tid][j] = pj;
        sum += pj;
      }
      l_s[tid] = l_s[tid] * alpha + sum;
      m_s[tid] = mx;
      a_s[tid] = alpha;
    }
    __syncthreads();
    for (int e = tid; e < G * D; e += kDecThreads) {
      const int r = e / D, d = e % D;
      float acc = o_s[r][d] * a_s[r];
      for (int j = 0; j < nt; ++j) acc += p_s[r][j] * v_s[j][d];
      o_s[r][d] = acc;
    }
    __syncthreads();
  }
  // partial of this chunk: [b][kvh][c][r] -> (m, l, o[D])
  float* out = part + ((static_cast<int64_t>(b) * Hkv + kvh) * n_chunks + c) * kDecMaxRows * (D + 2);
  for (int e = tid; e < G * (D + 2); e += kDecThreads) {
    const int r = e / (D + 2), d = e % (D + 2);
    out[r * (D + 2) + d] = d == 0 ? m_s[r] : (d == 1 ? l_s[r] : o_s[r][d - 2]);
  }
}

// One wave per (sample, token, q-head): merges the chunks.  Lanes take the
// chunks' (max, sum) for the overall maximum and sum; the output columns are
// then summed over the chunks with the weights broadcast from LDS (fixed order).
template <int D>
__global__ __launch_bounds__(kWave)
void decode_merge_kernel(const float* __restrict__ part, int n_new, int Hq, int Hkv, int n_chunks,
                         uint16_t* __restrict__ Od) {
  __shared__ float w_s[kDecMaxChunks];
  const int h = blockIdx.x, i = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x;
  const int g = Hq / Hkv;
  const int kvh = h / g, r = i * g + (h % g);
  const float* base = part + (static_cast<int64_t>(b) * Hkv + kvh) * n_chunks * kDecMaxRows * (D + 2);
  float M = -__builtin_inff();
  for (int c = lane; c < n_chunks; c += kWave) M = fmaxf(M, base[(c * kDecMaxRows + r) * (D + 2)]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, kWave));
  float L = 0.f;
  for (int c = lane; c < n_chunks; c += kWave) {
    const float* pc = base + (c * kDecMaxRows + r) * (D + 2);
    const float m = pc[0];
    const float w = m == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(m - M);
    w_s[c] = w;
    L += w * pc[1];
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) L += __shfl_xor(L, off, kWave);
  __syncthreads();
  float acc[D / kWave];
#pragma unroll
  for (int u = 0; u < D / kWave; ++u) acc[u] = 0.f;
  int c = 0;
  for (; c + 8 <= n_chunks; c += 8) {
    float v[8][D / kWave];
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int u = 0; u < D / kWave; ++u) v[t][u] = base[((c + t) * kDecMaxRows + r) * (D + 2) + 2 + u * kWave + lane];
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int u = 0; u < D / kWave; ++u) acc[u] += w_s[c + t] * v[t][u];
  }
  for (; c < n_chunks; ++c)
#pragma unroll
    for (int u = 0; u < D / kWave; ++u) acc[u] += w_s[c] * base[(c * kDecMaxRows + r) * (D + 2) + 2 + u * kWave + lane];
  const float inv = L > 0.f ? 1.f / L : 0.f;
  uint16_t* o = Od + ((static_cast<int64_t>(b) * n_new + i) * Hq + h) * D;
#pragma unroll
  for (int u = 0; u < D / kWave; ++u) {
    const __bf16 v = static_cast<__bf16>(acc[u] * inv);
    o[u * kWave + lane] = __builtin_bit_cast(uint16_t, v);
  }
}

}  // namespace

int decode_chunks(int B, int S_cap, int Hkv, int* chunk_out) {
  // enough workgroups to stream the cache on every CU (about two per CU), at
  // least one key tile per chunk
  const int64_t want = 512;
  int64_t per = (static_cast<int64_t>(S_cap) * Hkv * B + want - 1) / want;
  per = ((per + kDecTile - 1) / kDecTile) * kDecTile;
  if (per < kDecTile) per = kDecTile;
  const int64_t min_per = (S_cap + kDecMaxChunks - 1) / kDecMaxChunks;  // at most kDecMaxChunks chunks
  if (per < min_per) per = ((min_per + kDecTile - 1) / kDecTile) * kDecTile;
  *chunk_out = static_cast<int>(per);
  return static_cast<int>((S_cap + per - 1) / per);
}

size_t decode_workspace_bytes(int B, int S_cap, int Hkv, int D) {
  int chunk;
  const int n_chunks = decode_chunks(B, S_cap, Hkv, &chunk);
  return static_cast<size_t>(B) * Hkv * n_chunks * kDecMaxRows * (D + 2) * sizeof(float);
}

int decode_max_rows() { return kDecMaxRows; }

hipError_t launch_decode(int D, const void* Qd, const void* Kc, const void* Vc, const int32_t* n_kv, int B,
                         int S_cap, int n_new, int Hq, int Hkv, void* Od, float* part, hipStream_t stream) {
  int chunk;
  const int n_chunks = decode_chunks(B, S_cap, Hkv, &chunk);
  const float c = 1.4426950408889634f / sqrtf(static_cast<float>(D));
  const dim3 g1(n_chunks, Hkv, B), g2(Hq, n_new, B);
  auto q = static_cast<const uint16_t*>(Qd);
  auto k = static_cast<const uint16_t*>(Kc);
  auto v = static_cast<const uint16_t*>(Vc);
  auto o = static_cast<uint16_t*>(Od);
  if (D == 128) {
    hipLaunchKernelGGL(decode_chunk_kernel<128>, g1, dim3(kDecThreads), 0, stream, q, k, v, n_kv, S_cap, n_new, Hq,
                       Hkv, c, chunk, n_chunks, part);
    hipLaunchKernelGGL(decode_merge_kernel<128>, g2, dim3(kWave), 0, stream, part, n_new, Hq, Hkv, n_chunks, o);
  } else if (D == 64) {
    hipLaunchKernelGGL(decode_chunk_kernel<64>, g1, dim3(kDecThreads), 0, stream, q, k, v, n_kv, S_cap, n_new, Hq,
                       Hkv, c, chunk, n_chunks, part);
    hipLaunchKernelGGL(decode_merge_kernel<64>, g2, dim3(kWave), 0, stream, part, n_new, Hq, Hkv, n_chunks, o);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace dash
