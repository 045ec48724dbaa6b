/*
 * dash.h — C ABI of the DASH (Delta Attention Selective Halting) prefill path
 * for AMD Instinct MI355X (gfx950).
 *
 * Sources of the operations (web pages describing the method, cited by title
 * and section):
 *   [P1] "DASH：基于注意力增量的Transformer令牌压缩，实现长序列推理高效加速"
 *        (CSDN blog explainer): §2.1 Δattn definition, §2.3 single-shot
 *        decision, §3.1 algorithm steps, §3.2 parameters, §3.3 prefill loop
 *        sketch, §5.1/§5.2 engineering notes (no host/device syncs, efficient
 *        gathers).
 *   [P2] "DASH：通过注意力动态监测实现长上下文高效预填充" (zingnex forum):
 *        sections 层间更新动态监测 and 选择性停止机制 (threshold halting over
 *        consecutive layers; halted tokens keep their K/V).
 *
 * Conventions for every call
 *   - All tensor pointers are DEVICE pointers, 16-byte aligned, owned by the
 *     caller.  The library never allocates or frees device memory; scratch
 *     space comes from the caller's workspace (size from dash_workspace_size).
 *     A call uses its workspace until its last launch has run on its stream:
 *     calls that may overlap in time (other streams) must not share one.
 *     Nothing in a workspace needs to start at any particular value.
 *   - Every call is enqueued on `stream` (a hipStream_t passed as void*; NULL is
 *     the default stream) and returns without waiting.  Counts that depend on
 *     the data stay on the device (n_dev / n_out_dev), so no call performs a
 *     hidden host<->device synchronisation.
 *   - Arguments are validated before anything is enqueued.  An invalid call
 *     returns a nonzero dash_status, enqueues nothing, and leaves a message
 *     readable through dash_last_error().  A failed launch returns DASH_E_HIP.
 *     Faults during execution surface at the caller's next synchronisation.
 *     No C++ exception crosses this boundary.
 *   - `ctx` may be NULL (the current HIP device is used).
 *   - Layouts are dense and row-major:
 *       Q  [B, S, Hq,  D]      K, V [B, S, Hkv, D]   (token-major)
 *       O  [B, S, Hq*D]        (head h in columns h*D .. h*D+D-1)
 *       Wo [hidden, Hq*D]      out-major, like a linear layer's weight:
 *                              U[t][c] = sum_e O[t][e] * Wo[c][e]
 *       U  [B, S, hidden]      score [B, S] fp32
 *     Element type of Q, K, V, O, Wo and U is `dtype` (fp32 or bf16);
 *     arithmetic accumulates in fp32.
 *   - q-head h reads kv-head h / (Hq / Hkv); softmax scale is 1/sqrt(D).
 *   - Size limits checked by every call that takes a dash_shape: S <= 2^24,
 *     B * S <= 2^26, and one sample's K (and V), S * Hkv * D * element size
 *     bytes, below 4 GiB (the attention kernels address K and V through
 *     32-bit buffer offsets); DASH_E_SHAPE otherwise.
 */
#ifndef DASH_H
#define DASH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DASH_OK = 0,
  DASH_E_INVAL = 1,      /* null pointer, bad enum, out-of-range count */
  DASH_E_SHAPE = 2,      /* inconsistent or unsupported shape */
  DASH_E_DTYPE = 3,      /* unsupported element type for this call */
  DASH_E_ALIGN = 4,      /* pointer or row size not 16-byte aligned */
  DASH_E_WORKSPACE = 5,  /* workspace missing or too small */
  DASH_E_HIP = 6         /* HIP runtime error (launch, device query) */
} dash_status;

typedef enum { DASH_F32 = 0, DASH_BF16 = 1 } dash_dtype;
typedef enum { DASH_KV_ACTIVE = 0, DASH_KV_ALL = 1 } dash_kv_mode;
typedef enum { DASH_SEL_TOPK = 0, DASH_SEL_THRESHOLD = 1, DASH_SEL_ORDER_STAT = 2 } dash_sel_mode;
typedef enum { DASH_OP_ATTN_LAYER = 0, DASH_OP_SELECT = 1, DASH_OP_ATTN_ACTIVE = 2, DASH_OP_DECODE = 3 } dash_op;

/* Problem shape.  hidden is the width of U; Hq*D is the width of O. */
typedef struct {
  int B, S, Hq, Hkv, D, hidden;
  int dtype; /* dash_dtype */
} dash_shape;

/* Selection parameters.
 *   TOPK:        k kept per row.
 *   ORDER_STAT:  rank (1-based) of the order statistic among ascending scores.
 *   THRESHOLD:   tau (DEVICE pointer to one float), patience (consecutive
 *                layers below tau before a token halts), counters (DEVICE
 *                uint8 array indexed by original position) holding n_counters
 *                entries.  A row whose position lies outside [0, n_counters)
 *                is dropped: it is not emitted and no counter is touched.
 *   keep_first / keep_last: TOPK only (0 for the other modes): forced
 *                retention of the first f and last l positions of every row
 *                ([P1] §3.1 and §3.2: keep_first_n / keep_last_n).  k stays
 *                the total kept count (dash_keep_count gives it from the keep
 *                ratio) and 0 <= f + l <= k is required. */
typedef struct {
  int mode; /* dash_sel_mode */
  int k;
  int rank;
  const float* tau;
  int patience;
  uint8_t* counters;
  int keep_first, keep_last;
  int n_counters; /* THRESHOLD: entries of counters; unused otherwise */
} dash_sel;

/* Library context: remembers the device and its compute-unit count.
 * dash_create returns DASH_E_HIP when no device is usable. */
int dash_create(void** ctx, int device);
void dash_destroy(void* ctx);

/* Message of the last failed call on this host thread (library-owned). */
const char* dash_last_error(void);

/* Library version string. */
const char* dash_version(void);

/* Kept count of the one-shot policy ([P1] §3.1 step 3 and §3.2: K =
 * floor(keep * T) with keep = 1 - ρ; with forced retention of the first f =
 * keep_first and last l = keep_last tokens, K_eff = f + l + floor(keep * (T -
 * f - l))).  The product is formed in double precision and truncated, so
 * T = 131072, keep = 0.3 gives 39321.  Requires T >= 0, 0 <= keep <= 1 and
 * f, l >= 0 with f + l <= T (else DASH_E_INVAL and *k_out untouched). */
int dash_keep_count(int T, double keep, int keep_first, int keep_last, int* k_out);

/* Rank of the halting threshold of the selective-halting policy ([P2]
 * 层间更新动态监测: a token halts once its update stays below a preset
 * threshold): the nearest-rank pct-th percentile of n scores, rank =
 * ceil(pct * n / 100) in integer arithmetic and at least 1 (n = 65536,
 * pct = 30 gives 19661).  It is the `rank` of DASH_SEL_ORDER_STAT.  Requires
 * n >= 1 and 0 <= pct <= 100. */
int dash_percentile_rank(int n, int pct, int* rank_out);

/* Workspace bytes needed by `op` (dash_op) for shape s with up to n_max rows
 * (n_max is the sequence length for DASH_OP_ATTN_LAYER and the row capacity
 * for the others; for DASH_OP_SELECT the shape's B is the number of rows of
 * scores).  Returns 0 for an invalid request. */
size_t dash_workspace_size(void* ctx, int op, const dash_shape* s, int n_max);

/* a1 + a2: one full-length layer ([P1] §2.1, §3.1 steps 1-2).
 *   O = causal GQA softmax attention of Q, K, V          [B, S, Hq*D]
 *   U = O · Wo^T                                         [B, S, hidden]
 *   score[t] = ||U_t||_2 (fp32), taken from the fp32 accumulators before U is
 *   rounded to dtype.  score == NULL skips the score.
 * Supported: dtype bf16 with D in {64, 128}; dtype fp32 with D <= 128 and
 * D % 4 == 0 (reference-speed kernels).  hidden % 4 == 0; Hq % Hkv == 0.
 * The bf16 W_o GEMM picks 224- or 256-column tiles, whichever fills the
 * chip's compute units in fewer tile-widths of work.
 * Workspace: dash_workspace_size(DASH_OP_ATTN_LAYER, s, S). */
int dash_attn_layer(void* ctx, const dash_shape* s,
                    const void* Q, const void* K, const void* V, const void* Wo,
                    void* O, void* U, float* score,
                    void* ws, size_t ws_bytes, void* stream);

/* dash_attn_layer without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same arguments and results as dash_attn_layer (the
 * same kernels, bit-identical outputs) except that the Σu² partials of the
 * score live in a scratch array built into the library: 16 MiB per GPU, held
 * from the first call on that GPU until the process ends.  A score needs
 * ceil(hidden / 224) * B * S * 4 bytes of it (hidden 3584: B * S <= 262144);
 * larger calls with score != NULL return DASH_E_WORKSPACE and enqueue
 * nothing.  score == NULL needs no scratch.  The call allocates nothing.
 * Every call on one GPU shares that GPU's array: calls that overlap in time
 * on one GPU (several streams or host threads) race and must be serialised by
 * the caller.  Nothing in the array needs to start at zero. */
int dash_attn_layer_noalloc(void* ctx, const dash_shape* s,
                            const void* Q, const void* K, const void* V, const void* Wo,
                            void* O, void* U, float* score, void* stream);

/* a3 / a3': selection ([P1] §2.3 and §3.1 step 3; [P2] 层间更新动态监测).
 *   TOPK:       score [rows, n_max] → idx [rows, k]: the k positions with the
 *               largest score, ties to the lower position, NaN below every
 *               number, -0 == +0, written in ascending order.  If pos != NULL
 *               (rows == 1 only) the kept entries are pos[i] instead of i.
 *               n = n_max, or n = min(*n_dev, n_max) for rows == 1 when n_dev
 *               != NULL (a count left on the device by an earlier step); then
 *               min(k, n) positions are kept (f and l shrink likewise: f' =
 *               min(f, k'), l' = min(l, k' - f')) and idx entries past them
 *               are left untouched.  n_out_dev, if not NULL (rows == 1), gets
 *               the kept count.  With keep_first f and keep_last l, positions
 *               0..f-1 and n-l..n-1 are always kept and the other k - f - l
 *               are the top ones among positions f..n-l-1 under the same
 *               order; the output is still ascending.
 *   ORDER_STAT: rows == 1; n = *n_dev (or n_max); *tau_out (device) = the
 *               rank-th smallest of score[0..n) under the same order (NaN
 *               lowest), a zero returned as +0.  rank <= n is required when n
 *               comes from the device; otherwise tau_out is set to NaN.
 *   THRESHOLD:  rows == 1; n = *n_dev (or n_max); row i belongs to position
 *               p = pos[i] (pos == NULL ⇒ p = i; pos ascending).  For each row
 *               with 0 <= p < n_counters: counters[p] = score[i] < *tau ?
 *               counters[p] + 1 : 0 (saturating at 255) and the row stays
 *               active iff counters[p] < patience.  A NaN score is not below
 *               tau, so it resets the counter.  Surviving positions are written
 *               ascending to idx (capacity n_max) and their number to
 *               *n_out_dev (device int).  idx must not alias pos.
 * NaN status: when ws != NULL, row r's count of NaN scores (among the n it
 *   ranks or updates, forced ends included) is written to the int32 word r of
 *   ws; ws == NULL skips the count.
 * Workspace: dash_workspace_size(DASH_OP_SELECT, {B = rows, ...}, n_max)
 * bytes (4 per row, at least 256) when the NaN status is wanted.  For a
 * single row (rows == 1, no n_dev) whose middle (n_max - keep_first -
 * keep_last) exceeds 32768 scores, that size also covers the scratch of a
 * top-k spread over many workgroups (a chain of short launches), which runs
 * whenever the workspace is that large; with a smaller workspace (or none)
 * the row takes one workgroup.  The threshold step with n_max > 32768 uses
 * the same scratch the same way (two launches; a device count n_dev is
 * allowed).  Same results either way. */
int dash_select(void* ctx, const dash_sel* p, const float* score, const int32_t* pos,
                const int32_t* n_dev, int n_max, int rows,
                int32_t* idx, int32_t* n_out_dev, float* tau_out,
                void* ws, size_t ws_bytes, void* stream);

/* ---- Ragged batches ([P1] §5.1/§5.2: samples of one batch prune
 * independently; with different lengths and kept counts they are packed back
 * to back).  cu_* are DEVICE int32 prefix offsets with B + 1 entries
 * (cu[0] = 0, sample b owns rows cu[b] .. cu[b+1]-1 of the packed tensors);
 * their totals are passed from the host.  The kernels clamp every sample's
 * rows into those totals and capacities, so inconsistent offsets can give
 * wrong results but never out-of-bounds accesses. */

/* a1 + a2 for a packed batch: s->B samples, s->S = the longest sample,
 * cu_seqlens [B + 1], `total` = cu_seqlens[B] packed rows.  Q [total, Hq, D],
 * K, V [total, Hkv, D], O [total, Hq*D], U [total, hidden], score [total]:
 * causal attention within each sample, then the W_o GEMM and score over all
 * rows.  Workspace: dash_workspace_size(DASH_OP_ATTN_LAYER, {B = 1, S =
 * total, ...}, total). */
int dash_attn_layer_varlen(void* ctx, const dash_shape* s, const int32_t* cu_seqlens, int total,
                           const void* Q, const void* K, const void* V, const void* Wo, void* O, void* U,
                           float* score, void* ws, size_t ws_bytes, void* stream);

/* a3 for a packed batch (top-k only): sample b's n_b = cu_n[b+1] - cu_n[b]
 * scores (of n_total) keep k_b = cu_k[b+1] - cu_k[b] positions (k_b <= n_b;
 * with p->keep_first / keep_last applied per sample, f + l <= k_b), written
 * ascending to idx[cu_k[b] ..] as PACKED row indices (cu_n[b] + position in
 * the sample), so dash_compact / dash_compact_many gather them directly.
 * k_total = cu_k[B] is idx's capacity; max_n >= every n_b.  p->k is unused. */
int dash_select_ragged(void* ctx, const dash_sel* p, const float* score, int n_total, int B, const int32_t* cu_n,
                       const int32_t* cu_k, int max_n, int k_total, int32_t* idx, void* stream);

/* a5 for a packed batch: s->B samples, s->S = the most active rows of any
 * sample.  Qa [n_total, Hq, D] are the packed active queries (sample b's at
 * rows cu_q[b] .. cu_q[b+1]-1).  DASH_KV_ACTIVE: K, V are [n_total, Hkv, D],
 * compacted with the queries (cu_kv NULL or cu_q); q_pos unused.
 * DASH_KV_ALL: K, V are the full packed [kv_total, Hkv, D] with offsets
 * cu_kv (the batch's cu_seqlens) and q_pos [n_total] gives each query's packed
 * row (as dash_select_ragged writes it).  Oa [n_total, Hq*D]; if Wo != NULL,
 * Ua [n_total, hidden] and score [n_total] as in dash_attn_active.
 * Workspace: dash_workspace_size(DASH_OP_ATTN_ACTIVE, {B = 1, S = n_total,
 * ...}, n_total). */
int dash_attn_active_varlen(void* ctx, const dash_shape* s, const void* Qa, const int32_t* q_pos,
                            const int32_t* cu_q, int n_total, const void* K, const void* V, int kv_mode,
                            const int32_t* cu_kv, int kv_total, void* Oa, const void* Wo, void* Ua, float* score,
                            void* ws, size_t ws_bytes, void* stream);

/* Decode attention over a KV cache — the step after a (pruned) prefill ([P1]
 * §3.1 step 5, §5.1: the cache holds only the active tokens, so each decode
 * step reads less).  s->B samples, s->S = cache capacity (rows per sample),
 * s->Hq, s->Hkv, s->D (bf16 only, D in {64, 128}); s->hidden is unused.
 *   Qd [B, n_new, Hq, D]: the new tokens' queries.
 *   Kc, Vc [B, S, Hkv, D]: each sample's cache; sample b holds n_kv[b] rows
 *     (DEVICE int32 [B], clamped to S), its last n_new rows being the new
 *     tokens' own K/V, earlier rows the kept prefill tokens in position order.
 *   Od [B, n_new, Hq*D]: new token i sees cache rows 0 .. n_kv[b] - n_new + i.
 * Requires (Hq / Hkv) * n_new <= 32.  Split over the keys: workspace
 * dash_workspace_size(DASH_OP_DECODE, s, n_new). */
int dash_decode(void* ctx, const dash_shape* s, const void* Qd, int n_new, const void* Kc, const void* Vc,
                const int32_t* n_kv, void* Od, void* ws, size_t ws_bytes, void* stream);

/* Δattn from a given U ([P1] §2.1, §2.2: the score needs only U, so any
 * attention kernel can feed it): score[t] = ||U_t||_2 (fp32 sums of squares,
 * fixed order) for t < n, n = *n_dev (or n_max).  U is [n_max, hidden] of
 * dtype (bf16 or fp32), row-major, 16-byte aligned, hidden * element size a
 * multiple of 16 (hidden % 8 == 0 for bf16, % 4 for fp32).  score[t] for
 * t >= n is left untouched.  dash_attn_layer / dash_attn_active produce the
 * same score fused into their W_o GEMM; this call serves a U made elsewhere.
 * No workspace. */
int dash_score(void* ctx, const void* U, int dtype, int hidden, const int32_t* n_dev, int n_max, float* score,
               void* stream);

/* a4: compaction ([P1] §3.1 step 4, §3.3): Xa[r, :] = X[idx[r], :] for
 * r < n, n = *n_dev (or n_max).  X has S rows of row_bytes bytes (a multiple
 * of 16).  A row whose idx[r] lies outside [0, S) is not copied (its Xa row is
 * left as it was).  Rows of Xa at or beyond n are left untouched.  No
 * workspace. */
int dash_compact(void* ctx, const int32_t* idx, const int32_t* n_dev, int n_max,
                 const void* X, int S, size_t row_bytes, void* Xa, void* stream);

/* a4 for several tensors at once: the same gather for up to 4 tensors that
 * share one index list (a layer's Q, K and V at the kept positions), in one
 * launch.  For each j < count: items[j].Xa[r, :] = items[j].X[idx[r], :] for
 * r < n, with the rules of dash_compact (items[j].S rows of
 * items[j].row_bytes bytes, a multiple of 16; rows with idx[r] outside
 * [0, S) not copied).  `items` is a HOST array read during the call.
 * n_max times the summed row_bytes / 16 must stay below 2^31.  No workspace. */
typedef struct {
  const void* X;
  int S;
  size_t row_bytes;
  void* Xa;
} dash_gather;
int dash_compact_many(void* ctx, const int32_t* idx, const int32_t* n_dev, int n_max,
                      const dash_gather* items, int count, void* stream);

/* a4 for a batch of B samples of equal shape (same k per sample): for each
 * b < B, r < k and j < count, items[j].Xa[b*k + r, :] =
 * items[j].X[b*S_j + idx[b*k + r], :] with S_j = items[j].S rows per sample;
 * idx holds each sample's local positions (as dash_select writes them for
 * rows = B).  Other rules as dash_compact_many.  No workspace. */
int dash_compact_batch(void* ctx, const int32_t* idx, int B, int k, const dash_gather* items, int count,
                       void* stream);

/* a5: post-halt attention ([P1] §3.1 step 4 and §5.1; [P2] 选择性停止机制).
 *   Qa [B, n, Hq, D] are the active queries of B = s->B samples (n = n_max
 *   per sample; n = *n_dev allowed for B == 1 only), q_pos [B, n] their
 *   ascending original positions within the sample.
 *   DASH_KV_ACTIVE: K, V are [B, n, Hkv, D], compacted at the same positions
 *     (pruned tokens left the KV cache); q_pos may be NULL.
 *   DASH_KV_ALL: K, V are the full [B, S, Hkv, D] of this layer (halted
 *     tokens keep their K/V); q_pos is required.
 *   Key r is visible to query i iff pos(r) <= q_pos[i] (same sample).
 *   Oa [B, n, Hq*D].  If Wo != NULL: Ua = Oa · Wo^T [B, n, hidden], and
 *   score[b*n + i] = ||Ua_{b,i}||_2 when score != NULL.  Rows at or beyond n
 *   are left untouched.
 * Workspace: dash_workspace_size(DASH_OP_ATTN_ACTIVE, s, n_max) (covers the
 * B * n_max rows). */
int dash_attn_active(void* ctx, const dash_shape* s, const void* Qa, const int32_t* q_pos,
                     const int32_t* n_dev, int n_max, const void* K, const void* V, int kv_mode,
                     void* Oa, const void* Wo, void* Ua, float* score,
                     void* ws, size_t ws_bytes, void* stream);

/* a4 folded into a5 (the pages ask for gathers without needless tensor
 * copies: [P1] §3.3 closing note, §5.2 troubleshooting table): as
 * dash_attn_active, but the queries are not
 * compacted beforehand.  Q is the layer's full [B, S, Hq, D] (S = s->S) and
 * active query i of sample b is read from row q_rows[b * n_max + i] of that
 * sample (DEVICE int32 [B, n_max], values in [0, S); values outside are
 * clamped into it).  With DASH_KV_ALL, q_rows is normally q_pos itself; with
 * DASH_KV_ACTIVE only K and V need compacting (q_pos may be NULL).  Results
 * are identical to compacting Q at q_rows and calling dash_attn_active.
 * Errors and workspace as for dash_attn_active; DASH_E_INVAL if q_rows is
 * NULL. */
int dash_attn_active_gather(void* ctx, const dash_shape* s, const void* Q, const int32_t* q_rows,
                            const int32_t* q_pos, const int32_t* n_dev, int n_max, const void* K,
                            const void* V, int kv_mode, void* Oa, const void* Wo, void* Ua, float* score,
                            void* ws, size_t ws_bytes, void* stream);

/* Launch tracing (measurement support, not on the hot path).
 * dash_trace_start(capacity) creates 2*capacity HIP events on the current
 * device and starts recording: every kernel group the library enqueues is
 * bracketed by an event pair on its launch stream, until `capacity` groups
 * have been recorded or dash_trace_stop() is called.  dash_trace_read waits
 * for the recorded events and copies out, for up to `max` groups, the group
 * kind (dash_trace_op) and its elapsed milliseconds into host arrays; *n gets
 * the number copied.  Starting again discards earlier records.
 * dash_trace_select(op_mask) restricts recording to the kinds whose bit
 * (1u << dash_trace_op) is set, from the next launch on, so that a timed run
 * pays for the event pairs of the groups it measures only; dash_trace_start
 * resets the mask to every kind.  Not thread-safe with concurrent launches
 * from several host threads. */
typedef enum {
  DASH_TR_ATTN_LAYER = 0,   /* attention kernel of dash_attn_layer */
  DASH_TR_PROJ_LAYER = 1,   /* W_o GEMM (+ score finalize) of dash_attn_layer */
  DASH_TR_ATTN_ACTIVE = 2,  /* attention kernel of dash_attn_active */
  DASH_TR_PROJ_ACTIVE = 3,  /* W_o GEMM (+ score finalize) of dash_attn_active */
  DASH_TR_SELECT = 4,       /* selection kernel of dash_select */
  DASH_TR_COMPACT = 5,      /* gather kernel of dash_compact / dash_compact_many */
  DASH_TR_SCORE = 6,        /* row-norm kernel of dash_score */
  DASH_TR_DECODE = 7        /* chunk + merge kernels of dash_decode */
} dash_trace_op;

int dash_trace_start(int capacity);
int dash_trace_select(unsigned op_mask);
int dash_trace_stop(void);
int dash_trace_read(int* ops, float* ms, int max, int* n);

#ifdef __cplusplus
}
#endif

#endif /* DASH_H */
