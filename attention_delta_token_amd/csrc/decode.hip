// Decode attention over a (pruned) KV cache — the step after a DASH prefill:
// the cache keeps only the active tokens, which shortens every later decode
// step (CSDN explainer "DASH：基于注意力增量的Transformer令牌压缩，实现长序列推理
// 高效加速", §3.1 step 5 and §5.1).
//
// Flash-decoding split over the keys: one wave owns a chunk of the cache of
// one (sample, kv-head) and handles all g q-heads x n_new new tokens of that
// kv-head (the rows of the group) against it, one key per lane: a lane reads
// its key row with 16-byte loads and forms the rows' scores against queries
// broadcast from LDS; the softmax maximum and sum of each row are wave
// reductions; for P V each lane owns D/64 output columns, reads its columns
// of the value rows (coalesced) and takes P from a wave-private LDS table.
// The wave keeps fp32 partials (row maximum, sum of exponentials,
// unnormalised output) in the workspace, and a second kernel merges the
// chunks in a fixed order.  The work per byte of cache is tiny (VALU); what
// matters is that many waves stream the cache at once with no serial step.
#include <algorithm>

#include "dash_common.h"
#include "dash_kernels.h"

namespace dash {

namespace {

constexpr int kDecStep = kWave;       // keys per wave step (one per lane)
constexpr int kDecMaxRows = 32;        // g * n_new rows per kv-head
constexpr int kDecMaxChunks = 1024;    // key chunks per (sample, kv-head), at most
constexpr int kDecTargetGroups = 2048;  // chunk workgroups per launch the split aims at

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

constexpr int kDecWaves = 4;  // waves per chunk: each takes a quarter of the rows

// A workgroup of kDecWaves waves owns one chunk; wave w handles rows
// w * RPW .. w * RPW + RPW - 1 (rows past g * n_new carry zero queries and are
// not written).  Chunk c covers keys [c * steps * 64, (c + 1) * steps * 64).
// Every global load of a step is issued before the first use: the query rows
// (16-byte loads), this lane's key row (each wave reads it; the copies after
// the first come from L2) and a quarter of the step's value rows per wave
// (16-byte loads, parked in LDS for all waves as soon as they arrive).
template <int D, int RPW>
__global__ __launch_bounds__(kDecWaves * kWave)
void decode_chunk_kernel(const uint16_t* __restrict__ Qd, const uint16_t* __restrict__ Kc,
                         const uint16_t* __restrict__ Vc, const int32_t* __restrict__ n_kv_dev, int S_cap,
                         int n_new, int Hq, int Hkv, float c_log2, int steps, int n_chunks,
                         float* __restrict__ part) {
  constexpr int DL = D / kWave;                                    // output columns per lane
  constexpr int kQLoads = (RPW * D / 8 + kWave - 1) / kWave;       // 16-byte query loads per lane
  constexpr int kVLoads = kDecStep * D / 8 / (kDecWaves * kWave);  // 16-byte value loads per thread and step
  __shared__ __attribute__((aligned(16))) float q_s[kDecWaves][RPW][D];
  __shared__ __attribute__((aligned(16))) float p_s[kDecWaves][kDecStep][RPW < 4 ? 4 : RPW];
  __shared__ __attribute__((aligned(16))) uint16_t v_s[kDecStep][D];
  constexpr int kPS = RPW < 4 ? 4 : RPW;  // p_s row length (float4 writes)
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int c = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int g = Hq / Hkv;
  const int G = g * n_new;  // row r = token (r / g), q-head kvh * g + r % g
  const int r0 = wave * RPW;
  const int kv_ld = Hkv * D;
  const uint16_t* Kb = Kc + static_cast<int64_t>(b) * S_cap * kv_ld + static_cast<int64_t>(kvh) * D;
  const uint16_t* Vb = Vc + static_cast<int64_t>(b) * S_cap * kv_ld + static_cast<int64_t>(kvh) * D;
  // The key and value loads are bounded by the capacity S_cap (rows past the
  // sample's count are allocated), so they need not wait for the count; rows
  // at or past n_kv are masked once it has arrived.
  const int n_kv_raw = n_kv_dev[b];

  // this wave's query rows, pre-scaled into exp2 units (rows past G are zero)
  {
    u32x4 qq[kQLoads];
#pragma unroll
    for (int i = 0; i < kQLoads; ++i) {
      const int e = lane + kWave * i;
      const int rr = e / (D / 8), d0 = (e % (D / 8)) * 8;
      const int r = r0 + rr;
      qq[i] = u32x4{0u, 0u, 0u, 0u};
      if (rr < RPW && r < G) {
        const int tok = r / g, jh = r % g;
        qq[i] = *reinterpret_cast<const u32x4*>(Qd + ((static_cast<int64_t>(b) * n_new + tok) * Hq + kvh * g + jh) * D + d0);
      }
    }
#pragma unroll
    for (int i = 0; i < kQLoads; ++i) {
      const int e = lane + kWave * i;
      const int rr = e / (D / 8), d0 = (e % (D / 8)) * 8;
      if (rr < RPW) {
        float4 lo, hi;
        lo.x = __uint_as_float(qq[i][0] << 16) * c_log2;
        lo.y = __uint_as_float(qq[i][0] & 0xffff0000u) * c_log2;
        lo.z = __uint_as_float(qq[i][1] << 16) * c_log2;
        lo.w = __uint_as_float(qq[i][1] & 0xffff0000u) * c_log2;
        hi.x = __uint_as_float(qq[i][2] << 16) * c_log2;
        hi.y = __uint_as_float(qq[i][2] & 0xffff0000u) * c_log2;
        hi.z = __uint_as_float(qq[i][3] << 16) * c_log2;
        hi.w = __uint_as_float(qq[i][3] & 0xffff0000u) * c_log2;
        *reinterpret_cast<float4*>(&q_s[wave][rr][d0]) = lo;
        *reinterpret_cast<float4*>(&q_s[wave][rr][d0 + 4]) = hi;
      }
    }
  }
  float m_run[RPW], l_run[RPW], acc[RPW][DL];
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    m_run[r] = -__builtin_inff();
    l_run[r] = 0.f;
#pragma unroll
    for (int e = 0; e < DL; ++e) acc[r][e] = 0.f;
  }
#pragma unroll 1
  for (int st = 0; st < steps; ++st) {
    const int t0 = (c * steps + st) * kDecStep;
    if (t0 >= S_cap) break;  // the same for every wave of the workgroup
    const int t = t0 + lane;
    u32x4 kq[D / 8];
    const uint16_t* kr = Kb + static_cast<int64_t>(t < S_cap ? t : 0) * kv_ld;
#pragma unroll
    for (int dc = 0; dc < D / 8; ++dc) kq[dc] = *reinterpret_cast<const u32x4*>(kr + dc * 8);
    {
      u32x4 vq[kVLoads];
#pragma unroll
      for (int i = 0; i < kVLoads; ++i) {
        const int e = tid + kDecWaves * kWave * i;
        const int j = e / (D / 8), d0 = (e % (D / 8)) * 8;
        vq[i] = u32x4{0u, 0u, 0u, 0u};
        if (t0 + j < S_cap) vq[i] = *reinterpret_cast<const u32x4*>(Vb + static_cast<int64_t>(t0 + j) * kv_ld + d0);
      }
      const int n_kv = max(0, min(n_kv_raw, S_cap));
#pragma unroll
      for (int i = 0; i < kVLoads; ++i) {
        const int j = (tid + kDecWaves * kWave * i) / (D / 8);
        if (t0 + j >= n_kv) vq[i] = u32x4{0u, 0u, 0u, 0u};  // unused rows may hold anything
      }
      __syncthreads();  // every wave is done with the previous step's value rows
#pragma unroll
      for (int i = 0; i < kVLoads; ++i) {
        const int e = tid + kDecWaves * kWave * i;
        *reinterpret_cast<u32x4*>(&v_s[e / (D / 8)][(e % (D / 8)) * 8]) = vq[i];
      }
    }
    const int n_kv = max(0, min(n_kv_raw, S_cap));
    const bool valid = t < n_kv;
    float sc[RPW];
#pragma unroll
    for (int r = 0; r < RPW; ++r) sc[r] = 0.f;
    // (inside a branch: the scheduler then keeps the query reads next to their use)
    if (valid)
#pragma unroll
      for (int dc = 0; dc < D / 8; ++dc) {
        float kf[8];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          kf[2 * w] = __uint_as_float(kq[dc][w] << 16);
          kf[2 * w + 1] = __uint_as_float(kq[dc][w] & 0xffff0000u);
        }
#pragma unroll
        for (int r = 0; r < RPW; ++r) {
          const float4 qa = *reinterpret_cast<const float4*>(&q_s[wave][r][dc * 8]);
          const float4 qb = *reinterpret_cast<const float4*>(&q_s[wave][r][dc * 8 + 4]);
          float a = sc[r];
          a = fmaf(qa.x, kf[0], a);
          a = fmaf(qa.y, kf[1], a);
          a = fmaf(qa.z, kf[2], a);
          a = fmaf(qa.w, kf[3], a);
          a = fmaf(qb.x, kf[4], a);
          a = fmaf(qb.y, kf[5], a);
          a = fmaf(qb.z, kf[6], a);
          a = fmaf(qb.w, kf[7], a);
          sc[r] = a;
        }
      }
    // softmax of this step's keys, folded into the running row state
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      // key t is visible to row r iff t <= n_kv - n_new + r / g (its own token and the cache before it)
      const bool vis = valid && t <= n_kv - n_new + (r0 + r) / g;
      const float sr = vis ? sc[r] : -__builtin_inff();
      const float m_new = fmaxf(m_run[r], wave_max(sr));
      const bool none = m_new == -__builtin_inff();
      const float alpha = none ? 1.f : __builtin_amdgcn_exp2f(m_run[r] - m_new);
      const float pr = none ? 0.f : __builtin_amdgcn_exp2f(sr - m_new);
      l_run[r] = l_run[r] * alpha + wave_sum(pr);
      m_run[r] = m_new;
#pragma unroll
      for (int e = 0; e < DL; ++e) acc[r][e] *= alpha;
      sc[r] = pr;
    }
#pragma unroll
    for (int r = 0; r < kPS; r += 4)
      *reinterpret_cast<float4*>(&p_s[wave][lane][r]) = {sc[r], r + 1 < RPW ? sc[(r + 1) % RPW] : 0.f,
                                                          r + 2 < RPW ? sc[(r + 2) % RPW] : 0.f,
                                                          r + 3 < RPW ? sc[(r + 3) % RPW] : 0.f};
    __syncthreads();  // value rows from every wave; this wave's P
    // O += P V: lane owns columns lane*DL .. +DL-1
#pragma unroll 4
    for (int j = 0; j < kDecStep; ++j) {
      float v[DL];
      if constexpr (DL == 2) {
        const uint32_t w = *reinterpret_cast<const uint32_t*>(&v_s[j][lane * 2]);
        v[0] = __uint_as_float(w << 16);
        v[DL - 1] = __uint_as_float(w & 0xffff0000u);
      } else {
        v[0] = bf16_to_f32(v_s[j][lane]);
      }
#pragma unroll
      for (int r = 0; r < kPS; r += 4) {
        const float4 pj = *reinterpret_cast<const float4*>(&p_s[wave][j][r]);
        const float pv[4] = {pj.x, pj.y, pj.z, pj.w};
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (r + q < RPW)
#pragma unroll
            for (int e = 0; e < DL; ++e) acc[(r + q) % RPW][e] = fmaf(pv[q], v[e], acc[(r + q) % RPW][e]);
      }
    }
  }
  // partial of this chunk: [b][kvh][c][r] -> (m, l, o[D])
  float* out = part + ((static_cast<int64_t>(b) * Hkv + kvh) * n_chunks + c) * kDecMaxRows * (D + 2);
#pragma unroll
  for (int rr = 0; rr < RPW; ++rr) {
    const int r = r0 + rr;
    if (r < G) {
#pragma unroll
      for (int e = 0; e < DL; ++e) out[r * (D + 2) + 2 + lane * DL + e] = acc[rr][e];
      if (lane == 0) {
        out[r * (D + 2)] = m_run[rr];
        out[r * (D + 2) + 1] = l_run[rr];
      }
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
  const int per = (n_chunks + kMergeWaves - 1) / kMergeWaves;
  const int c_beg = min(n_chunks, wave * per), c_end = min(n_chunks, c_beg + per);
  float acc[DL];
#pragma unroll
  for (int u = 0; u < DL; ++u) acc[u] = 0.f;
  for (int c0 = c_beg; c0 < c_end; c0 += kBatch) {
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
    hipLaunchKernelGGL(kern, g1, dim3(kDecWaves * kWave), 0, stream, q, k, v, n_kv, S_cap, n_new, Hq, Hkv, c, steps,
                       n_chunks, part);
  };
  if (D == 128) {
    if (G <= 8)
      chunk_kernel(decode_chunk_kernel<128, 2>);
    else if (G <= 16)
      chunk_kernel(decode_chunk_kernel<128, 4>);
    else
      chunk_kernel(decode_chunk_kernel<128, 8>);
    hipLaunchKernelGGL(decode_merge_kernel<128>, g2, dim3(kMergeWaves * kWave), 0, stream, part, n_new, Hq, Hkv, n_chunks, o);
  } else if (D == 64) {
    if (G <= 8)
      chunk_kernel(decode_chunk_kernel<64, 2>);
    else if (G <= 16)
      chunk_kernel(decode_chunk_kernel<64, 4>);
    else
      chunk_kernel(decode_chunk_kernel<64, 8>);
    hipLaunchKernelGGL(decode_merge_kernel<64>, g2, dim3(kMergeWaves * kWave), 0, stream, part, n_new, Hq, Hkv, n_chunks, o);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace dash
