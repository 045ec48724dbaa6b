// Internal launchers of the DASH kernels (not part of the public ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dash {

// dtype: 0 = fp32, 1 = bf16.
hipError_t launch_attention(int dtype, int B, int D, const void* Q, const void* K, const void* V, void* O,
                            const int32_t* q_pos, const int32_t* n_dev, int n_q_max, int n_kv, int Hq, int Hkv,
                            int64_t q_bs, int64_t kv_bs, int64_t o_bs, int qp_bs, hipStream_t stream);

int wo_gemm_parts(int dtype, int N);
hipError_t launch_wo_gemm(int dtype, const void* A, const void* W, void* U, float* score, float* part,
                          const int32_t* m_dev, int M_max, int N, int K, hipStream_t stream);

hipError_t launch_topk(const float* score, int rows, int n, int k, int keep_first, int keep_last,
                       const int32_t* pos, int32_t* idx, hipStream_t stream);
hipError_t launch_order_stat(const float* score, const int32_t* n_dev, int n_max, int rank, float* tau_out,
                             hipStream_t stream);
hipError_t launch_threshold(const float* score, const int32_t* pos, const int32_t* n_dev, int n_max,
                            const float* tau, int patience, uint8_t* counters, int32_t* out, int32_t* n_out,
                            hipStream_t stream);

hipError_t launch_row_norm(int dtype, const void* U, const int32_t* n_dev, int n_max, int hidden, float* score,
                           hipStream_t stream);

// One tensor of a multi-tensor gather: Xa[r] = X[idx[r]], rows of row_bytes.
constexpr int kMaxGather = 4;
struct GatherItem {
  const void* X;
  int S;
  size_t row_bytes;
  void* Xa;
};
// per_sample > 0: idx holds per_sample local row indices per sample; row r
// reads X row (r / per_sample) * S + idx[r].
hipError_t launch_compact_many(const int32_t* idx, const int32_t* n_dev, int n_max, const GatherItem* items,
                               int count, hipStream_t stream, int per_sample = 0);
hipError_t launch_compact(const int32_t* idx, const int32_t* n_dev, int n_max, const void* X, int S,
                          size_t row_bytes, void* Xa, hipStream_t stream);

}  // namespace dash
