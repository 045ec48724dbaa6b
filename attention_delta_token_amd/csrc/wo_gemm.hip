// Output projection with the Δattn score fused into its epilogue.
//
// U = O · Wo^T (Wo stored out-major [hidden, Hq*D]) is the attention
// sublayer's update to the residual stream, and the token score is its row
// norm ||U_t||_2 — CSDN explainer "DASH：基于注意力增量的Transformer令牌压缩，
// 实现长序列推理高效加速", §2.1 (U and Δattn) and §2.2 (the norm costs next to
// nothing once U is produced).
//
// bf16 path: 128x128 output tile per 256-thread workgroup, K stepped by 64,
// operands double-buffered in LDS, v_mfma_f32_32x32x16_bf16 with fp32
// accumulation.  The tile is computed transposed (C^T = Wo_tile · O_tile^T) so
// that every lane holds a single output row: the row's sum of squares is then
// accumulated in registers straight from the fp32 accumulators, before U is
// rounded to bf16.  Each (row, 128-column tile) partial is written to the
// workspace and a finalize kernel adds the partials in a fixed order and takes
// the square root, so the score is bit-reproducible run to run (no atomics).
#include "dash_common.h"
#include "dash_kernels.h"

namespace dash {

namespace {

constexpr int kGemmThreads = 256;
constexpr int kBM = 128;           // rows of U (tokens)
constexpr int kBN = 128;           // columns of U (hidden channels)
constexpr int kBK = 64;            // contraction step
constexpr int kLdsRow = kBK + 8;   // padded LDS row (bf16 elements): 144 bytes
constexpr int kTileElems = kBM * kLdsRow;

__device__ __forceinline__ void gemm_load_tile(const uint16_t* __restrict__ base, int rows_valid, int ld,
                                               int k0, u32x4 (&r)[4]) {
  // 128 rows x 64 bf16 = 1024 chunks of 16 bytes; thread t takes chunks t, t+256, ...
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = threadIdx.x + i * kGemmThreads;
    const int row = c >> 3;
    const int kc = c & 7;
    if (row < rows_valid)
      r[i] = *reinterpret_cast<const u32x4*>(base + static_cast<size_t>(row) * ld + k0 + kc * 8);
    else
      r[i] = u32x4{0u, 0u, 0u, 0u};
  }
}

__device__ __forceinline__ void gemm_store_tile(uint16_t* lds, const u32x4 (&r)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = threadIdx.x + i * kGemmThreads;
    const int row = c >> 3;
    const int kc = c & 7;
    *reinterpret_cast<u32x4*>(lds + row * kLdsRow + kc * 8) = r[i];
  }
}

__global__ __launch_bounds__(kGemmThreads, 2)
void wo_gemm_bf16_kernel(const uint16_t* __restrict__ A, const uint16_t* __restrict__ W,
                         uint16_t* __restrict__ U, float* __restrict__ part,
                         const int32_t* __restrict__ m_dev, int M_max, int N, int K, int n_tiles_n,
                         int part_ld) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[4 * kTileElems];  // [stage][A|W]
  int M = m_dev ? *m_dev : M_max;
  if (M > M_max) M = M_max;
  const int n_tiles_m = (M_max + kBM - 1) / kBM;
  const int lid = xcd_remap(blockIdx.x, n_tiles_m * n_tiles_n);
  const int tn = lid % n_tiles_n;
  const int tm = lid / n_tiles_n;
  const int m0 = tm * kBM;
  const int n0 = tn * kBN;
  if (m0 >= M) return;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int wn = wave >> 1;  // 0..1 : 64-column half of the tile
  const int wm = wave & 1;   // 0..1 : 64-row half of the tile

  const uint16_t* Ab = A + static_cast<size_t>(m0) * K;
  const uint16_t* Wb = W + static_cast<size_t>(n0) * K;
  const int rows_a = min(kBM, M - m0);
  const int rows_w = min(kBN, N - n0);

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  u32x4 ra[4], rw[4];
  gemm_load_tile(Ab, rows_a, K, 0, ra);
  gemm_load_tile(Wb, rows_w, K, 0, rw);
  gemm_store_tile(lds, ra);
  gemm_store_tile(lds + kTileElems, rw);
  __syncthreads();

  const int KT = K / kBK;
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < KT;
    if (more) {
      gemm_load_tile(Ab, rows_a, K, (kt + 1) * kBK, ra);
      gemm_load_tile(Wb, rows_w, K, (kt + 1) * kBK, rw);
    }
    const uint16_t* la = lds + cur * 2 * kTileElems;
    const uint16_t* lw = la + kTileElems;
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      bf16x8 opw[2], opa[2];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
        opw[nb] = *reinterpret_cast<const bf16x8*>(lw + (wn * 64 + nb * 32 + l32) * kLdsRow + ks * 16 + hi * 8);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
        opa[mb] = *reinterpret_cast<const bf16x8*>(la + (wm * 64 + mb * 32 + l32) * kLdsRow + ks * 16 + hi * 8);
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) acc[nb][mb] = mfma32x32x16(opw[nb], opa[mb], acc[nb][mb]);
    }
    if (more) {
      uint16_t* nx = lds + (cur ^ 1) * 2 * kTileElems;
      gemm_store_tile(nx, ra);
      gemm_store_tile(nx + kTileElems, rw);
    }
    __syncthreads();
  }

  // ---- epilogue -----------------------------------------------------------
  // acc[nb][mb][r] = U[m][n] with m = m0 + wm*64 + mb*32 + l32,
  //                  n = n0 + wn*64 + nb*32 + (r/4)*8 + hi*4 + (r%4).
  float* red = reinterpret_cast<float*>(lds);            // [2 wn][128 m] partial sums
  uint16_t* ct = lds + 2 * kTileElems;                    // staging tile [128 m][kLdsC]
  constexpr int kLdsC = kBN + 8;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    float ss = 0.f;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int nl = wn * 64 + nb * 32 + (r >> 2) * 8 + hi * 4 + (r & 3);
        const float v = (n0 + nl < N) ? acc[nb][mb][r] : 0.f;
        ss += v * v;
      }
    ss += __shfl_xor(ss, 32, 64);
    const int ml = wm * 64 + mb * 32 + l32;
    if (hi == 0) red[wn * kBM + ml] = ss;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int nl = wn * 64 + nb * 32 + g * 8 + hi * 4;
        u32x2 pk;
        pk[0] = pack_bf16x2(acc[nb][mb][g * 4 + 0], acc[nb][mb][g * 4 + 1]);
        pk[1] = pack_bf16x2(acc[nb][mb][g * 4 + 2], acc[nb][mb][g * 4 + 3]);
        *reinterpret_cast<u32x2*>(ct + ml * kLdsC + nl) = pk;
      }
  }
  __syncthreads();
  if (part && tid < kBM) {
    const int m = m0 + tid;
    if (m < M) part[static_cast<size_t>(tn) * part_ld + m] = red[tid] + red[kBM + tid];
  }
  // Coalesced store of the bf16 tile: 128 rows x 16 chunks of 16 bytes.
#pragma unroll
  for (int i = 0; i < (kBM * kBN / 8) / kGemmThreads; ++i) {
    const int c = tid + i * kGemmThreads;
    const int row = c >> 4;
    const int cc = c & 15;
    const int m = m0 + row;
    const int n = n0 + cc * 8;
    if (m < M && n < N) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(ct + row * kLdsC + cc * 8);
      if (n + 8 <= N) {
        *reinterpret_cast<u32x4*>(U + static_cast<size_t>(m) * N + n) = v;
      } else {
        const uint16_t* e = reinterpret_cast<const uint16_t*>(&v);
        for (int j = 0; j < N - n; ++j) U[static_cast<size_t>(m) * N + n + j] = e[j];
      }
    }
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

__global__ __launch_bounds__(256)
void score_finalize_kernel(const float* __restrict__ part, int n_parts, int part_ld,
                           const int32_t* __restrict__ m_dev, int M_max, float* __restrict__ score) {
  int M = m_dev ? *m_dev : M_max;
  if (M > M_max) M = M_max;
  const int m = blockIdx.x * 256 + threadIdx.x;
  if (m >= M) return;
  float s = 0.f;
  for (int t = 0; t < n_parts; ++t) s += part[static_cast<size_t>(t) * part_ld + m];
  score[m] = sqrtf(s);
}

}  // namespace

int wo_gemm_parts(int dtype, int N) {
  const int bn = dtype == 1 ? kBN : kF32Tile;
  return (N + bn - 1) / bn;
}

hipError_t launch_wo_gemm(int dtype, const void* A, const void* W, void* U, float* score, float* part,
                          const int32_t* m_dev, int M_max, int N, int K, hipStream_t stream) {
  if (M_max <= 0) return hipSuccess;
  const int parts = wo_gemm_parts(dtype, N);
  if (dtype == 1) {
    const int tm = (M_max + kBM - 1) / kBM;
    hipLaunchKernelGGL(wo_gemm_bf16_kernel, dim3(tm * parts), dim3(kGemmThreads), 0, stream,
                       static_cast<const uint16_t*>(A), static_cast<const uint16_t*>(W),
                       static_cast<uint16_t*>(U), score ? part : nullptr, m_dev, M_max, N, K, parts, M_max);
  } else {
    hipLaunchKernelGGL(wo_gemm_f32_kernel, dim3(parts, (M_max + kF32Tile - 1) / kF32Tile), dim3(256), 0, stream,
                       static_cast<const float*>(A), static_cast<const float*>(W), static_cast<float*>(U),
                       score ? part : nullptr, m_dev, M_max, N, K, M_max);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !score) return e;
  hipLaunchKernelGGL(score_finalize_kernel, dim3((M_max + 255) / 256), dim3(256), 0, stream, part, parts, M_max,
                     m_dev, M_max, score);
  return hipGetLastError();
}

}  // namespace dash
