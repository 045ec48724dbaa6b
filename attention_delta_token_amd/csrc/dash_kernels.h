// Internal launchers of the DASH kernels (not part of the public ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dash {

// dtype: 0 = fp32, 1 = bf16.
// Where sample b's rows live.  Fixed batch (cu_q == nullptr): sample b starts
// b * q_bs / kv_bs / o_bs elements in, its query positions b * qp_bs entries
// in, and it has *n_dev (or n_q_max) queries.  Ragged (packed) batch: sample
// b's query rows are cu_q[b] .. cu_q[b+1]-1 and its key rows cu_kv[b] ..
// cu_kv[b+1]-1 of the packed tensors; query positions index the packed key
// rows, so a query's position within its sample is q_pos - cu_kv[b].  In both
// cases n_kv < 0 makes the key count follow the query count (keys compacted
// with the queries); a ragged batch otherwise takes it from cu_kv.
// q_rows (fixed batch only): query r of sample b reads row q_rows[b*qp_bs + r]
// of that sample's Q (clamped into [0, q_rows_n)) instead of row r, so the
// queries are gathered on load rather than compacted beforehand.
struct AttnBatch {
  int64_t q_bs = 0, kv_bs = 0, o_bs = 0;
  int qp_bs = 0;
  const int32_t* q_rows = nullptr;
  int q_rows_n = 0;
  const int32_t* cu_q = nullptr;
  const int32_t* cu_kv = nullptr;
  int q_total = 0, kv_total = 0;  // ragged: packed query / key rows; every sample is clamped into them

  // Moves the (restrict-qualified) tensor pointers to sample b and sets its
  // query count, key count and position base.
  template <class PQ, class PO, class PP, class PK>
  __device__ __forceinline__ void locate(int64_t b, const int32_t* n_dev, int n_q_max, int& n_kv, int q_ld,
                                         int kv_ld, PQ& Q, PO& O, PP& q_pos, PK& K, PK& V, int& n_q,
                                         int& pos_base) const {
    if (cu_q) {
      const int q_row0 = min(max(cu_q[b], 0), q_total);
      const int kv_row0 = min(max(cu_kv[b], 0), kv_total);
      n_q = max(0, min(min(cu_q[b + 1], q_total) - q_row0, n_q_max));
      n_kv = n_kv < 0 ? n_q : max(0, min(cu_kv[b + 1], kv_total) - kv_row0);
      pos_base = kv_row0;
      Q += static_cast<int64_t>(q_row0) * q_ld;
      O += static_cast<int64_t>(q_row0) * q_ld;
      if (q_pos) q_pos += q_row0;
      K += static_cast<int64_t>(kv_row0) * kv_ld;
      V += static_cast<int64_t>(kv_row0) * kv_ld;
    } else {
      n_q = n_dev ? *n_dev : n_q_max;
      if (n_q > n_q_max) n_q = n_q_max;
      if (n_kv < 0) n_kv = n_q;
      pos_base = 0;
      Q += b * q_bs;
      O += b * o_bs;
      if (q_pos) q_pos += b * qp_bs;
      K += b * kv_bs;
      V += b * kv_bs;
    }
  }
};

hipError_t launch_attention(int dtype, int B, int D, const void* Q, const void* K, const void* V, void* O,
                            const int32_t* q_pos, const int32_t* n_dev, int n_q_max, int n_kv, int Hq, int Hkv,
                            const AttnBatch& bt, hipStream_t stream);

int wo_gemm_parts(int dtype, int N);
hipError_t launch_wo_gemm(int dtype, const void* A, const void* W, void* U, float* score, float* part,
                          const int32_t* m_dev, int M_max, int N, int K, hipStream_t stream);

// n_dev (rows == 1 only): the row's score count is min(*n_dev, n) and at most
// that many are kept; n_out receives the kept count; nan_out[r] the number of
// NaN scores of row r (each may be null).
hipError_t launch_topk(const float* score, int rows, int n, int k, int keep_first, int keep_last,
                       const int32_t* pos, const int32_t* n_dev, int32_t* idx, int32_t* n_out, int32_t* nan_out,
                       hipStream_t stream);
// Single rows longer than 32768 scores (after the forced ends) over many
// workgroups; scratch of topk_multi_ws_bytes bytes (0: the row is too short).
size_t topk_multi_ws_bytes(int n_row, int keep_first, int keep_last);
hipError_t launch_topk_multi(const float* score, int n_row, int k_total, int keep_first, int keep_last,
                             const int32_t* pos, int32_t* idx, int32_t* n_out, int32_t* nan_out, void* scratch,
                             hipStream_t stream);
// Ragged top-k: sample b's scores are cu_n[b] .. cu_n[b+1]-1 of `score`
// (n_total entries); it keeps cu_k[b+1] - cu_k[b] of them, written as packed
// row indices to idx[cu_k[b] ..] (capacity k_cap); max_n bounds every
// sample's length.
hipError_t launch_topk_ragged(const float* score, int n_total, int B, const int32_t* cu_n, const int32_t* cu_k,
                              int max_n, int k_cap, int keep_first, int keep_last, int32_t* idx, hipStream_t stream);
hipError_t launch_order_stat(const float* score, const int32_t* n_dev, int n_max, int rank, float* tau_out,
                             int32_t* nan_out, hipStream_t stream);
// Rows whose position lies outside [0, n_counters) are dropped.
hipError_t launch_threshold(const float* score, const int32_t* pos, const int32_t* n_dev, int n_max,
                            const float* tau, int patience, uint8_t* counters, int n_counters, int32_t* out,
                            int32_t* n_out, int32_t* nan_out, hipStream_t stream);
// The same step over many workgroups for more than 32768 rows (capacity),
// with topk_multi_ws_bytes(n_max, 0, 0) bytes of scratch.
hipError_t launch_threshold_multi(const float* score, const int32_t* pos, const int32_t* n_dev, int n_max,
                                  const float* tau, int patience, uint8_t* counters, int n_counters, int32_t* out,
                                  int32_t* n_out, int32_t* nan_out, void* scratch, hipStream_t stream);

hipError_t launch_row_norm(int dtype, const void* U, const int32_t* n_dev, int n_max, int hidden, float* score,
                           hipStream_t stream);

// Decode attention (bf16, D in {64, 128}): g * n_new <= decode_max_rows().
int decode_chunks(int B, int S_cap, int Hkv, int* steps_out);
size_t decode_workspace_bytes(int B, int S_cap, int Hkv, int D);
int decode_max_rows();
hipError_t launch_decode(int D, const void* Qd, const void* Kc, const void* Vc, const int32_t* n_kv, int B,
                         int S_cap, int n_new, int Hq, int Hkv, void* Od, float* part, hipStream_t stream);

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
