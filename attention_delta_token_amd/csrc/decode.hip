// Decode attention over a (pruned) KV cache — the step after a DASH prefill:
// the cache keeps only the active tokens, which shortens every later decode
// step (CSDN explainer "DASH：基于注意力增量的Transformer令牌压缩，实现长序列推理
// 高效加速", §3.1 step 5 and §5.1).
//
// Flash-decoding split over the keys: one wave owns a chunk of the cache of
// one (sample, kv-head) and handles all g q-heads x n_new new tokens of that
// kv-head (the rows of the group, up to 32) against it on the matrix cores
// (see decode_mfma_kernel).  The wave keeps fp32 partials (row maximum, sum of
// exponentials, unnormalised output) in the workspace, and a second kernel
// merges the chunks in a fixed order.  What matters is that many waves stream
// the cache at once: the arithmetic per byte of cache is small.
#include <algorithm>

#include "dash_common.h"
#include "dash_kernels.h"

namespace dash {

namespace {

constexpr int kDecStep = 64;          // keys per chunk step (two 32-key sub-steps)
constexpr int kDecMaxRows = 32;        // g * n_new rows per kv-head
constexpr int kDecMaxChunks = 1024;    // key chunks per (sample, kv-head), at most
constexpr int kDecTargetGroups = 1024;  // chunk workgroups per launch the split aims at

// Wave-wide max / sum in registers: a rotate butterfly inside each 16-lane
// row (DPP row_ror 8, 4, 2, 1), then the four row results through readlane,
// combined in a fixed order so every lane gets the same value.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}

__device__ __forceinline__ float lane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp<0x128>(v));
  v = fmaxf(v, dpp<0x124>(v));
  v = fmaxf(v, dpp<0x122>(v));
  v = fmaxf(v, dpp<0x121>(v));
  return fmaxf(fmaxf(lane_f(v, 0), lane_f(v, 16)), fmaxf(lane_f(v, 32), lane_f(v, 48)));
}

__device__ __forceinline__ float wave_sum(float v) {
  v += dpp<0x128>(v);
  v += dpp<0x124>(v);
  v += dpp<0x122>(v);
  v += dpp<0x121>(v);
  return (lane_f(v, 0) + lane_f(v, 16)) + (lane_f(v, 32) + lane_f(v, 48));
}

// ---------------------------------------------------------------------------
// Chunk kernel: one wave per chunk holds all g * n_new rows of its (sample,
// kv-head) (up to 32, one per lane pair) and runs each 32-key sub-step as two
// small products on v_mfma_f32_32x32x16_bf16:
//   S^T = K Q^T (keys x rows; K read straight from memory in operand layout,
//   Q pre-scaled into exp2 units once), the online softmax per row (a lane
//   and its partner 32 lanes away hold one row), P rounded to bf16 in the
//   accumulator's key order, and O^T += V^T P^T with V staged in LDS (rows
//   XOR-swizzled by 16-byte chunk) and read transposed (ds_read_b64_tr_b16)
//   in the key order P arrives in.  Rows past g * n_new compute on zero
//   queries and are not written.  The partials have the layout the merge
//   kernel reads.
// ---------------------------------------------------------------------------
typedef short dec_i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t dec_u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ dec_i16x4 dec_read_tr16(const unsigned char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) dec_i16x4*)(p));
}

// Slot of 16-byte chunk c of V row r in LDS: the four rows x 64 bytes one
// transposing read fetches for 32 lanes land in distinct banks.
template <int D>
__device__ __forceinline__ int dec_v_slot(int r, int c) {
  constexpr int kRowBytes = D * 2, kChunks = kRowBytes / 16, kRowsPerLine = 256 / kRowBytes;
  return c ^ (4 * ((r / kRowsPerLine) % (kChunks / 4)));
}

template <int D>
__global__ __launch_bounds__(kWave, 2)  // at least two waves per SIMD
void decode_mfma_kernel(const uint16_t* __restrict__ Qd, const uint16_t* __restrict__ Kc,
                        const uint16_t* __restrict__ Vc, const int32_t* __restrict__ n_kv_dev, int S_cap,
                        int n_new, int Hq, int Hkv, float c_log2, int steps, int n_chunks,
                        float* __restrict__ part) {
  constexpr int kRowBytes = D * 2;
  constexpr int kChunks = kRowBytes / 16;                 // 16-byte chunks per key row
  constexpr int kSub = 32;                                // keys per sub-step (one MFMA key block)
  constexpr int kVLoads = kSub * kChunks / kWave;         // 16-byte V loads per lane and sub-step
  __shared__ __attribute__((aligned(16))) unsigned char vt[kSub * kRowBytes];
  const int lane = threadIdx.x, l32 = lane & 31, hi = lane >> 5;
  const int c = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int g = Hq / Hkv;
  const int G = g * n_new;  // row r = token (r / g), q-head kvh * g + r % g
  const int kv_ld = Hkv * D;
  const uint16_t* Kb = Kc + static_cast<int64_t>(b) * S_cap * kv_ld + static_cast<int64_t>(kvh) * D;
  const uint16_t* Vb = Vc + static_cast<int64_t>(b) * S_cap * kv_ld + static_cast<int64_t>(kvh) * D;
  const int n_kv = max(0, min(n_kv_dev[b], S_cap));
  const int row = l32;
  // keys t <= lim are visible to this lane's row (its own token and the cache before it)
  const int lim = min(n_kv - n_new + row / g, n_kv - 1);

  // B operand of S^T = K Q^T: this lane's row, d = 16 ks + 8 hi .. +7, times log2(e)/sqrt(D)
  bf16x8 qreg[D / 16];
  {
    u32x4 raw[D / 16];
    const int tok = row / g, jh = row % g;
    const uint16_t* qp = Qd + ((static_cast<int64_t>(b) * n_new + (row < G ? tok : 0)) * Hq + kvh * g + jh) * D + hi * 8;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) raw[ks] = *reinterpret_cast<const u32x4*>(qp + ks * 16);
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float lo = row < G ? __uint_as_float(raw[ks][w] << 16) * c_log2 : 0.f;
        const float up = row < G ? __uint_as_float(raw[ks][w] & 0xffff0000u) * c_log2 : 0.f;
        qreg[ks][2 * w] = static_cast<__bf16>(lo);
        qreg[ks][2 * w + 1] = static_cast<__bf16>(up);
      }
  }
  // transposed V operand offsets (lane-dependent part), as P's key order requires
  const int tj = lane & 15, tgrp = (lane >> 4) & 1;
  int voffs[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    const int vr = (tj >> 2) + 4 * hi;
    const int e = db * 32 + 16 * tgrp + 4 * (tj & 3);
    voffs[db] = vr * kRowBytes + 16 * dec_v_slot<D>(vr, e >> 3) + 2 * (e & 7);
  }

  f32x16 o[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[i][r] = 0.f;
  float m_run = -__builtin_inff(), l_run = 0.f;  // l_run: this half-wave's keys
#pragma unroll 1
  for (int sst = 0; sst < 2 * steps; ++sst) {
    const int t0 = c * steps * kDecStep + sst * kSub;
    if (t0 >= S_cap) break;
    // every load of the sub-step issued before the first use (addresses
    // clamped into the cache; rows at or past n_kv are masked or zeroed below)
    bf16x8 kop[D / 16];
    {
      const int t = min(t0 + l32, S_cap - 1);
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks)
        kop[ks] = *reinterpret_cast<const bf16x8*>(Kb + static_cast<int64_t>(t) * kv_ld + ks * 16 + hi * 8);
    }
    u32x4 vq[kVLoads];
#pragma unroll
    for (int i = 0; i < kVLoads; ++i) {
      const int e = lane + kWave * i;
      const int t = min(t0 + e / kChunks, S_cap - 1);
      vq[i] = *reinterpret_cast<const u32x4*>(Vb + static_cast<int64_t>(t) * kv_ld + (e % kChunks) * 8);
    }
    f32x16 s;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) s = mfma32x32x16(kop[ks], qreg[ks], s);
    // V rows of the sub-step into LDS (rows past n_kv as zeros: cache rows there may hold anything)
#pragma unroll
    for (int i = 0; i < kVLoads; ++i) {
      const int e = lane + kWave * i;
      const int vr = e / kChunks;
      const u32x4 v = t0 + vr < n_kv ? vq[i] : u32x4{0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4*>(vt + vr * kRowBytes + 16 * dec_v_slot<D>(vr, e % kChunks)) = v;
    }
    // online softmax of this sub-step's keys, in exp2 units
    float mx = -__builtin_inff();
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int t = t0 + (r >> 2) * 8 + hi * 4 + (r & 3);
      s[r] = t <= lim ? s[r] : -__builtin_inff();
      mx = fmaxf(mx, s[r]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    const bool none = m_new == -__builtin_inff();
    const float alpha = none ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
    const float mref = none ? 0.f : m_new;
    m_run = m_new;
#pragma unroll
    for (int i = 0; i < D / 32; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[i][r] *= alpha;
    u32x4 pk[2];
    float ps = 0.f;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
      for (int t2 = 0; t2 < 4; ++t2) {
        const float p0 = __builtin_amdgcn_exp2f(s[8 * sub + 2 * t2] - mref);
        const float p1 = __builtin_amdgcn_exp2f(s[8 * sub + 2 * t2 + 1] - mref);
        ps += p0 + p1;
        pk[sub][t2] = pack_bf16x2(p0, p1);
      }
    }
    l_run = l_run * alpha + ps;
    // O^T += V^T P^T (the V writes above precede these reads in the wave's LDS order)
#pragma unroll
    for (int stp = 0; stp < 2; ++stp)
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const dec_i16x4 lo = dec_read_tr16(vt + voffs[db] + (16 * stp) * kRowBytes);
        const dec_i16x4 up = dec_read_tr16(vt + voffs[db] + (16 * stp + 8) * kRowBytes);
        const u32x4 av = u32x4{__builtin_bit_cast(dec_u32x2, lo)[0], __builtin_bit_cast(dec_u32x2, lo)[1],
                               __builtin_bit_cast(dec_u32x2, up)[0], __builtin_bit_cast(dec_u32x2, up)[1]};
        o[db] = mfma32x32x16(__builtin_bit_cast(bf16x8, av), __builtin_bit_cast(bf16x8, pk[stp]), o[db]);
      }
  }
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  // partial of this chunk: [b][kvh][c][r] -> (m, l, o[D]); o^T element (d, row) with
  // d = 32 db + 8 (r / 4) + 4 hi + r % 4
  if (row < G) {
    float* out = part + (((static_cast<int64_t>(b) * Hkv + kvh) * n_chunks + c) * kDecMaxRows + row) * (D + 2);
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) out[2 + db * 32 + (r >> 2) * 8 + hi * 4 + (r & 3)] = o[db][r];
    if (hi == 0) {
      out[0] = m_run;
      out[1] = l_tot;
    }
  }
}

// One workgroup of kMergeWaves waves per (sample, token, q-head) merges the
// chunks.  Threads load every chunk's (max, sum) in one pass for the overall
// maximum and sum (workgroup reductions in a fixed order); wave w then sums the
// output columns of its contiguous range of chunks, 32 chunks' loads in flight
// at a time, with the weights from LDS, and the waves' sums are added in wave
// order: the result does not depend on timing.
constexpr int kMergeWaves = 8;

template <int D>
__global__ __launch_bounds__(kMergeWaves * kWave)
void decode_merge_kernel(const float* __restrict__ part, int n_new, int Hq, int Hkv, int n_chunks,
                         uint16_t* __restrict__ Od) {
  constexpr int DL = D / kWave;
  constexpr int NT = kMergeWaves * kWave;
  constexpr int kPer = (kDecMaxChunks + NT - 1) / NT;  // chunks per thread in the (max, sum) pass
  constexpr int kBatch = 32;                           // chunks per column batch
  __shared__ float w_s[kDecMaxChunks];
  __shared__ float red[2][kMergeWaves];
  __shared__ float acc_s[kMergeWaves][D];
  const int h = blockIdx.x, i = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g = Hq / Hkv;
  const int kvh = h / g, r = i * g + (h % g);
  const float* base = part + (static_cast<int64_t>(b) * Hkv + kvh) * n_chunks * kDecMaxRows * (D + 2);
  float mc[kPer], lc[kPer];
#pragma unroll
  for (int t = 0; t < kPer; ++t) {
    const int c = tid + NT * t;
    mc[t] = -__builtin_inff();
    lc[t] = 0.f;
    if (c < n_chunks) {
      const float* pc = base + (c * kDecMaxRows + r) * (D + 2);
      mc[t] = pc[0];
      lc[t] = pc[1];
    }
  }
  // This wave's contiguous run of chunks; the output columns of its first
  // kBatch chunks are loaded together with the (max, sum) pass (chunk indices
  // clamped into the existing chunks, their weights zeroed below).
  const int per = (n_chunks + kMergeWaves - 1) / kMergeWaves;
  const int c_beg = min(n_chunks, wave * per), c_end = min(n_chunks, c_beg + per);
  float v0[kBatch][DL];
#pragma unroll
  for (int t = 0; t < kBatch; ++t)
#pragma unroll
    for (int u = 0; u < DL; ++u)
      v0[t][u] = base[(min(c_beg + t, n_chunks - 1) * kDecMaxRows + r) * (D + 2) + 2 + u * kWave + lane];
  float M = mc[0];
#pragma unroll
  for (int t = 1; t < kPer; ++t) M = fmaxf(M, mc[t]);
  M = wave_max(M);
  if (lane == 0) red[0][wave] = M;
  __syncthreads();
  M = red[0][0];
#pragma unroll
  for (int w = 1; w < kMergeWaves; ++w) M = fmaxf(M, red[0][w]);
  float L = 0.f;
#pragma unroll
  for (int t = 0; t < kPer; ++t) {
    const int c = tid + NT * t;
    const float w = mc[t] == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(mc[t] - M);
    if (c < n_chunks) w_s[c] = w;
    L += w * lc[t];
  }
  L = wave_sum(L);
  if (lane == 0) red[1][wave] = L;
  __syncthreads();  // weights and per-wave sums visible to every wave
  L = 0.f;
#pragma unroll
  for (int w = 0; w < kMergeWaves; ++w) L += red[1][w];
  float acc[DL];
#pragma unroll
  for (int u = 0; u < DL; ++u) acc[u] = 0.f;
#pragma unroll
  for (int t = 0; t < kBatch; ++t) {
    const float w = c_beg + t < c_end ? w_s[c_beg + t] : 0.f;
#pragma unroll
    for (int u = 0; u < DL; ++u) acc[u] = fmaf(w, v0[t][u], acc[u]);
  }
  for (int c0 = c_beg + kBatch; c0 < c_end; c0 += kBatch) {
    float v[kBatch][DL];
#pragma unroll
    for (int t = 0; t < kBatch; ++t)
#pragma unroll
      for (int u = 0; u < DL; ++u)
        v[t][u] = c0 + t < c_end ? base[((c0 + t) * kDecMaxRows + r) * (D + 2) + 2 + u * kWave + lane] : 0.f;
#pragma unroll
    for (int t = 0; t < kBatch; ++t) {
      const float w = c0 + t < c_end ? w_s[c0 + t] : 0.f;
#pragma unroll
      for (int u = 0; u < DL; ++u) acc[u] = fmaf(w, v[t][u], acc[u]);
    }
  }
#pragma unroll
  for (int u = 0; u < DL; ++u) acc_s[wave][u * kWave + lane] = acc[u];
  __syncthreads();
  if (wave == 0) {
    const float inv = L > 0.f ? 1.f / L : 0.f;
    uint16_t* o = Od + ((static_cast<int64_t>(b) * n_new + i) * Hq + h) * D;
#pragma unroll
    for (int u = 0; u < DL; ++u) {
      float sum = acc_s[0][u * kWave + lane];
#pragma unroll
      for (int w = 1; w < kMergeWaves; ++w) sum += acc_s[w][u * kWave + lane];
      const __bf16 ov = static_cast<__bf16>(sum * inv);
      o[u * kWave + lane] = __builtin_bit_cast(uint16_t, ov);
    }
  }
}

}  // namespace

int decode_chunks(int B, int S_cap, int Hkv, int* steps_out) {
  // one workgroup per 64 keys while that gives at most about kDecTargetGroups
  // chunk workgroups in all (between 8 and kDecMaxChunks per (sample,
  // kv-head)); longer caches give each workgroup several 64-key steps, which
  // keeps the merge of the chunks short
  const int64_t groups = static_cast<int64_t>(B > 0 ? B : 1) * (Hkv > 0 ? Hkv : 1);
  const int64_t cap = std::max<int64_t>(8, std::min<int64_t>(kDecMaxChunks, kDecTargetGroups / groups));
  const int64_t tiles = (static_cast<int64_t>(S_cap) + kDecStep - 1) / kDecStep;
  const int64_t steps = (tiles + cap - 1) / cap;
  *steps_out = static_cast<int>(steps < 1 ? 1 : steps);
  return static_cast<int>((tiles + *steps_out - 1) / *steps_out);
}

size_t decode_workspace_bytes(int B, int S_cap, int Hkv, int D) {
  int chunk;
  const int n_chunks = decode_chunks(B, S_cap, Hkv, &chunk);
  return static_cast<size_t>(B) * Hkv * n_chunks * kDecMaxRows * (D + 2) * sizeof(float);
}

int decode_max_rows() { return kDecMaxRows; }

hipError_t launch_decode(int D, const void* Qd, const void* Kc, const void* Vc, const int32_t* n_kv, int B,
                         int S_cap, int n_new, int Hq, int Hkv, void* Od, float* part, hipStream_t stream) {
  int steps;
  const int n_chunks = decode_chunks(B, S_cap, Hkv, &steps);
  const float c = 1.4426950408889634f / sqrtf(static_cast<float>(D));
  const dim3 g1(n_chunks, Hkv, B), g2(Hq, n_new, B);
  const int G = (Hq / Hkv) * n_new;
  if (G > kDecMaxRows) return hipErrorInvalidValue;
  auto q = static_cast<const uint16_t*>(Qd);
  auto k = static_cast<const uint16_t*>(Kc);
  auto v = static_cast<const uint16_t*>(Vc);
  auto o = static_cast<uint16_t*>(Od);
  auto chunk_kernel = [&](auto kern) {
    hipLaunchKernelGGL(kern, g1, dim3(kWave), 0, stream, q, k, v, n_kv, S_cap, n_new, Hq, Hkv, c, steps, n_chunks,
                       part);
  };
  if (D == 128) {
    chunk_kernel(decode_mfma_kernel<128>);
    hipLaunchKernelGGL(decode_merge_kernel<128>, g2, dim3(kMergeWaves * kWave), 0, stream, part, n_new, Hq, Hkv,
                       n_chunks, o);
  } else if (D == 64) {
    chunk_kernel(decode_mfma_kernel<64>);
    hipLaunchKernelGGL(decode_merge_kernel<64>, g2, dim3(kMergeWaves * kWave), 0, stream, part, n_new, Hq, Hkv,
                       n_chunks, o);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace dash
