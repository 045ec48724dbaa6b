// C ABI of the DASH prefill path: argument validation, workspace sizing,
// error reporting and kernel dispatch.  Every entry point validates its
// arguments with plain host code before any HIP call, so invalid calls
// enqueue nothing (and can be exercised without a GPU).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <exception>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/dash.h"
#include "dash_kernels.h"

namespace {

thread_local std::string g_last_error;

struct Ctx {
  int device;
  int cu_count;
};

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(DASH_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

size_t align_up(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// ---- shape checks shared by the attention entry points ---------------------
int check_shape(const dash_shape* s, bool need_b1) {
  if (!s) return fail(DASH_E_INVAL, "shape is NULL");
  if (s->dtype != DASH_F32 && s->dtype != DASH_BF16) return fail(DASH_E_DTYPE, "dtype %d unsupported", s->dtype);
  if (s->B < 1 || s->S < 1 || s->Hq < 1 || s->Hkv < 1 || s->D < 1 || s->hidden < 1)
    return fail(DASH_E_SHAPE, "B, S, Hq, Hkv, D and hidden must be >= 1");
  if (need_b1 && s->B != 1) return fail(DASH_E_SHAPE, "this call supports B == 1 only");
  if (s->Hq % s->Hkv != 0) return fail(DASH_E_SHAPE, "Hq (%d) must be a multiple of Hkv (%d)", s->Hq, s->Hkv);
  if (s->S > (1 << 24)) return fail(DASH_E_SHAPE, "S above 2^24 unsupported");
  if (static_cast<int64_t>(s->B) * s->S > (1ll << 26)) return fail(DASH_E_SHAPE, "B*S above 2^26 unsupported");
  if (s->Hq > 1024 || s->D > 1024 || s->hidden > (1 << 20)) return fail(DASH_E_SHAPE, "head count or width too large");
  // the attention kernels address one sample's K and V with 32-bit buffer offsets
  const int64_t esz = s->dtype == DASH_BF16 ? 2 : 4;
  if (static_cast<int64_t>(s->S) * s->Hkv * s->D * esz >= (1ll << 32))
    return fail(DASH_E_SHAPE, "one sample's K (S * Hkv * D * element size = %lld bytes) must stay below 4 GiB",
                static_cast<long long>(static_cast<int64_t>(s->S) * s->Hkv * s->D * esz));
  if (s->dtype == DASH_BF16) {
    if (s->D != 64 && s->D != 128) return fail(DASH_E_SHAPE, "bf16 path supports D in {64, 128}, got %d", s->D);
    if (s->hidden % 8 != 0) return fail(DASH_E_SHAPE, "bf16 path needs hidden %% 8 == 0, got %d", s->hidden);
  } else {
    if (s->D != 32 && s->D != 64 && s->D != 128)
      return fail(DASH_E_SHAPE, "fp32 path supports D in {32, 64, 128}, got %d", s->D);
    if (s->hidden % 4 != 0) return fail(DASH_E_SHAPE, "fp32 path needs hidden %% 4 == 0, got %d", s->hidden);
  }
  return DASH_OK;
}

size_t score_ws_bytes(const dash_shape* s, int64_t rows) {
  return align_up(static_cast<size_t>(dash::wo_gemm_parts(s->dtype, s->hidden)) * static_cast<size_t>(rows) *
                  sizeof(float));
}

int check_ptrs(std::initializer_list<std::pair<const void*, const char*>> ps) {
  for (auto& p : ps) {
    if (!p.first) return fail(DASH_E_INVAL, "%s is NULL", p.second);
    if (!aligned16(p.first)) return fail(DASH_E_ALIGN, "%s is not 16-byte aligned", p.second);
  }
  return DASH_OK;
}

// ---- launch tracing ----------------------------------------------------------
std::mutex g_tr_mu;
std::vector<hipEvent_t> g_tr_ev;  // 2 per record
std::vector<int> g_tr_op;
int g_tr_n = 0;
bool g_tr_on = false;
uint32_t g_tr_mask = ~0u;  // dash_trace_op kinds that are recorded

void trace_release() {
  for (hipEvent_t e : g_tr_ev) (void)hipEventDestroy(e);
  g_tr_ev.clear();
  g_tr_op.clear();
  g_tr_n = 0;
}

// Records the opening event of a traced kernel group; returns its slot or -1.
int trace_open(int op, hipStream_t st) {
  if (!g_tr_on) return -1;
  std::lock_guard<std::mutex> lk(g_tr_mu);
  if (!g_tr_on || g_tr_n >= static_cast<int>(g_tr_op.size()) || !((g_tr_mask >> op) & 1u)) return -1;
  const int slot = g_tr_n++;
  g_tr_op[slot] = op;
  (void)hipEventRecord(g_tr_ev[2 * slot], st);
  return slot;
}

void trace_close(int slot, hipStream_t st) {
  if (slot >= 0) (void)hipEventRecord(g_tr_ev[2 * slot + 1], st);
}

// a1 + a2 on validated arguments; part holds the Σu² partials (score != NULL).
int attn_layer_launch(const dash_shape* s, const void* Q, const void* K, const void* V, const void* Wo, void* O,
                      void* U, float* score, float* part, hipStream_t st) {
  const int64_t rows = static_cast<int64_t>(s->B) * s->S;
  const int64_t qd = static_cast<int64_t>(s->Hq) * s->D;
  const int64_t kvd = static_cast<int64_t>(s->Hkv) * s->D;
  int tr = trace_open(DASH_TR_ATTN_LAYER, st);
  dash::AttnBatch bt;
  bt.q_bs = s->S * qd;
  bt.kv_bs = s->S * kvd;
  bt.o_bs = s->S * qd;
  hipError_t e = dash::launch_attention(s->dtype, s->B, s->D, Q, K, V, O, nullptr, nullptr, s->S, s->S, s->Hq,
                                        s->Hkv, bt, st);
  trace_close(tr, st);
  if (e != hipSuccess) return hip_fail(e, "attention launch");
  tr = trace_open(DASH_TR_PROJ_LAYER, st);
  e = dash::launch_wo_gemm(s->dtype, O, Wo, U, score, part, nullptr, static_cast<int>(rows), s->hidden,
                           static_cast<int>(qd), st);
  trace_close(tr, st);
  if (e != hipSuccess) return hip_fail(e, "projection launch");
  return DASH_OK;
}

// ---- built-in scratch for dash_attn_layer_noalloc -----------------------------
// Every GPU the library runs on holds its own copy of this array until the
// process ends.  Host code never uses the array's name as a device address:
// the address of each device's copy is looked up once per device (with that
// device current) and kept in g_scratch_ptr.
constexpr size_t kScratchBytes = size_t(16) << 20;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_address(float** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(DASH_E_HIP, "device %d beyond the scratch table", dev);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(DASH_E_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = p;
  }
  *out = static_cast<float*>(g_scratch_ptr[dev]);
  return DASH_OK;
}

}  // namespace

extern "C" {

int dash_trace_start(int capacity) {
  try {
    if (capacity < 1 || capacity > (1 << 20)) return fail(DASH_E_INVAL, "trace capacity %d out of range", capacity);
    std::lock_guard<std::mutex> lk(g_tr_mu);
    g_tr_on = false;
    trace_release();
    g_tr_ev.resize(2 * static_cast<size_t>(capacity));
    for (size_t i = 0; i < g_tr_ev.size(); ++i) {
      hipError_t e = hipEventCreate(&g_tr_ev[i]);
      if (e != hipSuccess) {
        g_tr_ev.resize(i);
        trace_release();
        return hip_fail(e, "hipEventCreate");
      }
    }
    g_tr_op.assign(static_cast<size_t>(capacity), -1);
    g_tr_mask = ~0u;
    g_tr_on = true;
    return DASH_OK;
  } catch (...) {
    return fail(DASH_E_INVAL, "unexpected host exception");
  }
}

int dash_trace_select(unsigned op_mask) {
  std::lock_guard<std::mutex> lk(g_tr_mu);
  g_tr_mask = op_mask;
  return DASH_OK;
}

int dash_trace_stop(void) {
  std::lock_guard<std::mutex> lk(g_tr_mu);
  g_tr_on = false;
  return DASH_OK;
}

int dash_trace_read(int* ops, float* ms, int max, int* n) {
  try {
    if (!n || max < 0 || (max > 0 && (!ops || !ms))) return fail(DASH_E_INVAL, "bad trace_read arguments");
    std::lock_guard<std::mutex> lk(g_tr_mu);
    const int m = g_tr_n < max ? g_tr_n : max;
    for (int i = 0; i < m; ++i) {
      hipError_t e = hipEventSynchronize(g_tr_ev[2 * i + 1]);
      if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
      float t = 0.f;
      e = hipEventElapsedTime(&t, g_tr_ev[2 * i], g_tr_ev[2 * i + 1]);
      if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
      ops[i] = g_tr_op[i];
      ms[i] = t;
    }
    *n = m;
    return DASH_OK;
  } catch (...) {
    return fail(DASH_E_INVAL, "unexpected host exception");
  }
}

const char* dash_last_error(void) { return g_last_error.c_str(); }

const char* dash_version(void) { return "dash-mi355x 0.2.0 (gfx950)"; }

int dash_keep_count(int T, double keep, int keep_first, int keep_last, int* k_out) {
  if (!k_out) return fail(DASH_E_INVAL, "k_out is NULL");
  if (T < 0) return fail(DASH_E_INVAL, "T = %d must be >= 0", T);
  if (!(keep >= 0.0 && keep <= 1.0)) return fail(DASH_E_INVAL, "keep ratio %g outside [0, 1]", keep);
  if (keep_first < 0 || keep_last < 0 || static_cast<int64_t>(keep_first) + keep_last > T)
    return fail(DASH_E_INVAL, "forced counts keep_first %d + keep_last %d must lie in [0, T = %d]", keep_first,
                keep_last, T);
  const int rest = T - keep_first - keep_last;
  const int chosen = static_cast<int>(std::floor(keep * static_cast<double>(rest)));
  *k_out = keep_first + keep_last + (chosen < rest ? chosen : rest);
  return DASH_OK;
}

int dash_percentile_rank(int n, int pct, int* rank_out) {
  if (!rank_out) return fail(DASH_E_INVAL, "rank_out is NULL");
  if (n < 1) return fail(DASH_E_INVAL, "n = %d must be >= 1", n);
  if (pct < 0 || pct > 100) return fail(DASH_E_INVAL, "percentile %d outside [0, 100]", pct);
  const int64_t r = (static_cast<int64_t>(pct) * n + 99) / 100;  // ceil(pct * n / 100)
  *rank_out = r < 1 ? 1 : static_cast<int>(r);
  return DASH_OK;
}

int dash_create(void** ctx, int device) {
  try {
    if (!ctx) return fail(DASH_E_INVAL, "ctx is NULL");
    *ctx = nullptr;
    int n = 0;
    hipError_t e = hipGetDeviceCount(&n);
    if (e != hipSuccess) return hip_fail(e, "hipGetDeviceCount");
    if (device < 0 || device >= n) return fail(DASH_E_HIP, "device %d not present (%d devices)", device, n);
    int cus = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device);
    if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");
    *ctx = new Ctx{device, cus};
    return DASH_OK;
  } catch (...) {
    return fail(DASH_E_INVAL, "unexpected host exception");
  }
}

void dash_destroy(void* ctx) { delete static_cast<Ctx*>(ctx); }

size_t dash_workspace_size(void* /*ctx*/, int op, const dash_shape* s, int n_max) {
  try {
    switch (op) {
      case DASH_OP_ATTN_LAYER:
        if (check_shape(s, false) != DASH_OK) return 0;
        return score_ws_bytes(s, static_cast<int64_t>(s->B) * s->S);
      case DASH_OP_ATTN_ACTIVE:
        if (check_shape(s, false) != DASH_OK || n_max < 0) return 0;
        return score_ws_bytes(s, static_cast<int64_t>(s->B) * n_max);
      case DASH_OP_SELECT:  // one int32 NaN count per row; for one row longer than 32768 scores, the
                            // scratch of its multi-workgroup top-k
        if (!s || s->B < 1 || s->B > (1 << 20) || n_max < 0) return 0;
        return align_up(static_cast<size_t>(s->B) * sizeof(int32_t)) +
               (s->B == 1 ? dash::topk_multi_ws_bytes(n_max, 0, 0) : 0);
      case DASH_OP_DECODE:
        if (check_shape(s, false) != DASH_OK || n_max < 1) return 0;
        return align_up(dash::decode_workspace_bytes(s->B, s->S, s->Hkv, s->D));
      default:
        return 0;
    }
  } catch (...) {
    return 0;
  }
}

int dash_attn_layer(void* /*ctx*/, const dash_shape* s, const void* Q, const void* K, const void* V,
                    const void* Wo, void* O, void* U, float* score, void* ws, size_t ws_bytes, void* stream) {
  try {
    int rc = check_shape(s, false);
    if (rc) return rc;
    rc = check_ptrs({{Q, "Q"}, {K, "K"}, {V, "V"}, {Wo, "Wo"}, {O, "O"}, {U, "U"}});
    if (rc) return rc;
    const int64_t rows = static_cast<int64_t>(s->B) * s->S;
    if (score) {
      if (!aligned16(score)) return fail(DASH_E_ALIGN, "score is not 16-byte aligned");
      const size_t need = score_ws_bytes(s, rows);
      if (!ws || ws_bytes < need) return fail(DASH_E_WORKSPACE, "workspace needs %zu bytes, got %zu", need, ws ? ws_bytes : 0);
      if (!aligned16(ws)) return fail(DASH_E_ALIGN, "workspace is not 16-byte aligned");
    }
    return attn_layer_launch(s, Q, K, V, Wo, O, U, score, static_cast<float*>(ws), static_cast<hipStream_t>(stream));
  } catch (...) {
    return fail(DASH_E_INVAL, "unexpected host exception");
  }
}

int dash_attn_layer_noalloc(void* /*ctx*/, const dash_shape* s, const void* Q, const void* K, const void* V,
                            const void* Wo, void* O, void* U, float* score, void* stream) {
  try {
    int rc = check_shape(s, false);
    if (rc) return rc;
    rc = check_ptrs({{Q, "Q"}, {K, "K"}, {V, "V"}, {Wo, "Wo"}, {O, "O"}, {U, "U"}});
    if (rc) return rc;
    float* part = nullptr;
    if (score) {
      if (!aligned16(score)) return fail(DASH_E_ALIGN, "score is not 16-byte aligned");
      const size_t need = score_ws_bytes(s, static_cast<int64_t>(s->B) * s->S);
      if (need > kScratchBytes)
        return fail(DASH_E_WORKSPACE, "the score partials need %zu bytes; the built-in scratch holds %zu", need,
                    static_cast<size_t>(kScratchBytes));
      rc = scratch_address(&part);
      if (rc) return rc;
    }
    return attn_layer_launch(s, Q, K, V, Wo, O, U, score, part, static_cast<hipStream_t>(stream));
  } catch (...) {
    return fail(DASH_E_INVAL, "unexpected host exception");
  }
}

int dash_select(void* /*ctx*/, const dash_sel* p, const float* score, const int32_t* pos, const int32_t* n_dev,
                int n_max, int rows, int32_t* idx, int32_t* n_out_dev, float* tau_out, void* ws, size_t ws_bytes,
                void* stream) {
  try {
    if (!p) return fail(DASH_E_INVAL, "selection parameters are NULL");
    if (p->mode != DASH_SEL_TOPK && (p->keep_first != 0 || p->keep_last != 0))
      return fail(DASH_E_INVAL, "keep_first / keep_last apply to top-k only and must be 0 here");
    if (n_max < 0 || n_max > (1 << 30)) return fail(DASH_E_INVAL, "n_max %d out of range", n_max);
    if (rows < 1 || rows > (1 << 20)) return fail(DASH_E_INVAL, "rows %d out of range", rows);
    // NaN status: one int32 per row in the workspace, when one is given
    int32_t* nan_out = nullptr;
    if (ws) {
      const size_t need = align_up(static_cast<size_t>(rows) * sizeof(int32_t));
      if (ws_bytes < need) return fail(DASH_E_WORKSPACE, "workspace needs %zu bytes, got %zu", need, ws_bytes);
      if (!aligned4(ws)) return fail(DASH_E_ALIGN, "workspace is not 4-byte aligned");
      nan_out = static_cast<int32_t*>(ws);
    }
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e = hipSuccess;
    int tr = -1;
    switch (p->mode) {
      case DASH_SEL_TOPK: {
        if (p->k < 0 || p->k > n_max) return fail(DASH_E_INVAL, "k = %d outside [0, %d]", p->k, n_max);
        if (p->keep_first < 0 || p->keep_last < 0 ||
            static_cast<int64_t>(p->keep_first) + p->keep_last > p->k)
          return fail(DASH_E_INVAL, "forced counts keep_first %d + keep_last %d must lie in [0, k = %d]",
                      p->keep_first, p->keep_last, p->k);
        if ((n_dev || n_out_dev) && rows != 1)
          return fail(DASH_E_INVAL, "a device count (n_dev / n_out_dev) is supported for a single row only");
        if (pos && rows != 1) return fail(DASH_E_INVAL, "pos is supported for a single row only");
        if (static_cast<int64_t>(rows) * n_max > (1ll << 31) - 1)
          return fail(DASH_E_INVAL, "rows * n_max too large");
        if (p->k == 0 && !n_out_dev && !nan_out) return DASH_OK;
        if (!score && n_max > 0) return fail(DASH_E_INVAL, "score is NULL");
        if (!idx && p->k > 0) return fail(DASH_E_INVAL, "idx is NULL");
        if (n_max == 0 && !n_out_dev && !nan_out) return DASH_OK;
        tr = trace_open(DASH_TR_SELECT, st);
        // a single long row runs over many workgroups when the workspace holds
        // their scratch (after the status word)
        const size_t multi = (rows == 1 && !n_dev && p->k - p->keep_first - p->keep_last > 0)
                                 ? dash::topk_multi_ws_bytes(n_max, p->keep_first, p->keep_last)
                                 : 0;
        const size_t status_bytes = align_up(sizeof(int32_t));
        if (multi > 0 && ws && ws_bytes >= status_bytes + multi)
          e = dash::launch_topk_multi(score, n_max, p->k, p->keep_first, p->keep_last, pos, idx, n_out_dev, nan_out,
                                      static_cast<unsigned char*>(ws) + status_bytes, st);
        else
          e = dash::launch_topk(score, rows, n_max, p->k, p->keep_first, p->keep_last, pos, n_dev, idx, n_out_dev,
                                nan_out, st);
        break;
      }
      case DASH_SEL_ORDER_STAT: {
        if (rows != 1) return fail(DASH_E_INVAL, "order statistic supports one row");
        if (!score || !tau_out) return fail(DASH_E_INVAL, "score and tau_out are required");
        if (p->rank < 1) return fail(DASH_E_INVAL, "rank must be >= 1");
        if (!n_dev && p->rank > n_max) return fail(DASH_E_INVAL, "rank %d exceeds n %d", p->rank, n_max);
        tr = trace_open(DASH_TR_SELECT, st);
        e = dash::launch_order_stat(score, n_dev, n_max, p->rank, tau_out, nan_out, st);
        break;
      }
      case DASH_SEL_THRESHOLD: {
        if (rows != 1) return fail(DASH_E_INVAL, "threshold selection supports one row");
        if (!p->tau || !p->counters) return fail(DASH_E_INVAL, "tau and counters are required");
        if (p->n_counters < 1) return fail(DASH_E_INVAL, "n_counters = %d must be >= 1", p->n_counters);
        if (p->patience < 1 || p->patience > 255) return fail(DASH_E_INVAL, "patience must be in [1, 255]");
        if (!idx || !n_out_dev) return fail(DASH_E_INVAL, "idx and n_out_dev are required");
        if (n_max > 0 && !score) return fail(DASH_E_INVAL, "score is NULL");
        if (!pos && n_max > p->n_counters)
          return fail(DASH_E_INVAL, "without pos, rows are positions: n_max %d exceeds n_counters %d", n_max,
                      p->n_counters);
        if (pos && static_cast<const void*>(pos) == static_cast<const void*>(idx))
          return fail(DASH_E_INVAL, "idx must not alias pos");
        tr = trace_open(DASH_TR_SELECT, st);
        // more than 32768 rows run over many workgroups when the workspace holds
        // their scratch (after the status word)
        const size_t multi = dash::topk_multi_ws_bytes(n_max, 0, 0);
        const size_t status_bytes = align_up(sizeof(int32_t));
        if (multi > 0 && ws && ws_bytes >= status_bytes + multi)
          e = dash::launch_threshold_multi(score, pos, n_dev, n_max, p->tau, p->patience, p->counters, p->n_counters,
                                           idx, n_out_dev, nan_out, static_cast<unsigned char*>(ws) + status_bytes, st);
        else
          e = dash::launch_threshold(score, pos, n_dev, n_max, p->tau, p->patience, p->counters, p->n_counters, idx,
                                     n_out_dev, nan_out, st);
        break;
      }
      default:
        return fail(DASH_E_INVAL, "selection mode %d unknown", p->mode);
    }
    trace_close(tr, st);
    if (e != hipSuccess) return hip_fail(e, "selection launch");
    return DASH_OK;
  } catch (...) {
    return fail(DASH_E_INVAL, "unexpected host exception");
  }
}

int dash_compact(void* /*ctx*/, const int32_t* idx, const int32_t* n_dev, int n_max, const void* X, int S,
                 size_t row_bytes, void* Xa, void* stream) {
  try {
    if (n_max < 0) return fail(DASH_E_INVAL, "n_max must be >= 0");
    if (S < 0) return fail(DASH_E_INVAL, "S must be >= 0");
    if (row_bytes == 0 || row_bytes % 16 != 0) return fail(DASH_E_ALIGN, "row_bytes must be a positive multiple of 16");
    if (n_max == 0) return DASH_OK;
    int rc = check_ptrs({{X, "X"}, {Xa, "Xa"}});
    if (rc) return rc;
    if (!idx) return fail(DASH_E_INVAL, "idx is NULL");
    if (static_cast<uint64_t>(n_max) * (row_bytes / 16) >= (1ull << 31))
      return fail(DASH_E_INVAL, "n_max * row_bytes too large");
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int tr = trace_open(DASH_TR_COMPACT, st);
    hipError_t e = dash::launch_compact(idx, n_dev, n_max, X, S, row_bytes, Xa, st);
    trace_close(tr, st);
    if (e != hipSuccess) return hip_fail(e, "compaction launch");
    return DASH_OK;
  } catch (...) {
    return fail(DASH_E_INVAL, "unexpected host exception");
  }
}

int dash_attn_layer_varlen(void* /*ctx*/, const dash_shape* s, const int32_t* cu_seqlens, int total,
                           const void* Q, const void* K, const void* V, const void* Wo, void* O, void* U,
                           float* score, void* ws, size_t ws_bytes, void* stream) {
  try {
    int rc = check_shape(s, false);
    if (rc) return rc;
    if (total < 0 || static_cast<int64_t>(total) > static_cast<int64_t>(s->B) * s->S)
      return fail(DASH_E_SHAPE, "total %d outside [0, B * S]", total);
    if (total == 0) return DASH_OK;
    rc = check_ptrs({{Q, "Q"}, {K, "K"}, {V, "V"}, {Wo, "Wo"}, {O, "O"}, {U, "U"}});
    if (rc) return rc;
    if (!cu_seqlens) return fail(DASH_E_INVAL, "cu_seqlens is NULL");
    if (score) {
      if (!aligned16(score)) return fail(DASH_E_ALIGN, "score is not 16-byte aligned");
      const size_t need = score_ws_bytes(s, total);
      if (!ws || ws_bytes < need) return fail(DASH_E_WORKSPACE, "workspace needs %zu bytes, got %zu", need, ws ? ws_bytes : 0);
      if (!aligned16(ws)) return fail(DASH_E_ALIGN, "workspace is not 16-byte aligned");
    }
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int64_t qd = static_cast<int64_t>(s->Hq) * s->D;
    dash::AttnBatch bt;
    bt.cu_q = cu_seqlens;
    bt.cu_kv = cu_seqlens;
    bt.q_total = total;
    bt.kv_total = total;
    int tr = trace_open(DASH_TR_ATTN_LAYER, st);
    hipError_t e = dash::launch_attention(s->dtype, s->B, s->D, Q, K, V, O, nullptr, nullptr, s->S, 0, s->Hq,
                                          s->Hkv, bt, st);
    trace_close(tr, st);
    if (e != hipSuccess) return hip_fail(e, "attention launch");
    tr = trace_open(DASH_TR_PROJ_LAYER, st);
    e = dash::launch_wo_gemm(s->dtype, O, Wo, U, score, static_cast<float*>(ws), nullptr, total, s->hidden,
                             static_cast<int>(qd), st);
    trace_close(tr, st);
    if (e != hipSuccess) return hip_fail(e, "projection launch");
    return DASH_OK;
  } catch (...) {
    return fail(DASH_E_INVAL, "unexpected host exception");
  }
}

int dash_attn_active_varlen(void* /*ctx*/, const dash_shape* s, const void* Qa, const int32_t* q_pos,
                            const int32_t* cu_q, int n_total, const void* K, const void* V, int kv_mode,
                            const int32_t* cu_kv, int kv_total, void* Oa, const void* Wo, void* Ua, float* score,
                            void* ws, size_t ws_bytes, void* stream) {
  try {
    int rc = check_shape(s, false);
    if (rc) return rc;
    if (kv_mode != DASH_KV_ACTIVE && kv_mode != DASH_KV_ALL) return fail(DASH_E_INVAL, "kv_mode %d unknown", kv_mode);
    if (n_total < 0 || static_cast<int64_t>(n_total) > static_cast<int64_t>(s->B) * s->S)
      return fail(DASH_E_SHAPE, "n_total %d outside [0, B * S]", n_total);
    if (n_total == 0) return DASH_OK;
    rc = check_ptrs({{Qa, "Qa"}, {K, "K"}, {V, "V"}, {Oa, "Oa"}});
    if (rc) return rc;
    if (!cu_q) return fail(DASH_E_INVAL, "cu_q is NULL");
    if (kv_mode == DASH_KV_ALL && (!q_pos || !cu_kv)) return fail(DASH_E_INVAL, "kv_mode ALL needs q_pos and cu_kv");
    if (kv_mode == DASH_KV_ALL && (kv_total < 1 || kv_total > (1 << 26)))
      return fail(DASH_E_SHAPE, "kv_total %d outside [1, 2^26]", kv_total);
    if (kv_mode == DASH_KV_ACTIVE && cu_kv && cu_kv != cu_q)
      return fail(DASH_E_INVAL, "kv_mode ACTIVE keeps the keys with the queries (cu_kv must be NULL or cu_q)");
    if (Wo) {
      rc = check_ptrs({{Wo, "Wo"}, {Ua, "Ua"}});
      if (rc) return rc;
      if (score) {
        if (!aligned16(score)) return fail(DASH_E_ALIGN, "score is not 16-byte aligned");
        const size_t need = score_ws_bytes(s, n_total);
        if (!ws || ws_bytes < need) return fail(DASH_E_WORKSPACE, "workspace needs %zu bytes, got %zu", need, ws ? ws_bytes : 0);
        if (!aligned16(ws)) return fail(DASH_E_ALIGN, "workspace is not 16-byte aligned");
      }
    } else if (Ua || score) {
      return fail(DASH_E_INVAL, "Ua / score need Wo");
    }
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int64_t qd = static_cast<int64_t>(s->Hq) * s->D;
    dash::AttnBatch bt;
    bt.cu_q = cu_q;
    bt.cu_kv = kv_mode == DASH_KV_ACTIVE ? cu_q : cu_kv;
    bt.q_total = n_total;
    bt.kv_total = kv_mode == DASH_KV_ACTIVE ? n_total : kv_total;
    const int n_kv = kv_mode == DASH_KV_ACTIVE ? -1 : 0;  // ACTIVE: keys follow the queries; ALL: from cu_kv
    const int32_t* qp = kv_mode == DASH_KV_ALL ? q_pos : nullptr;
    int tr = trace_open(DASH_TR_ATTN_ACTIVE, st);
    hipError_t e = dash::launch_attention(s->dtype, s->B, s->D, Qa, K, V, Oa, qp, nullptr, s->S, n_kv, s->Hq,
                                          s->Hkv, bt, st);
    trace_close(tr, st);
    if (e != hipSuccess) return hip_fail(e, "attention launch");
    if (Wo) {
      tr = trace_open(DASH_TR_PROJ_ACTIVE, st);
      e = dash::launch_wo_gemm(s->dtype, Oa, Wo, Ua, score, static_cast<float*>(ws), nullptr, n_total, s->hidden,
                               static_cast<int>(qd), st);
      trace_close(tr, st);
      if (e != hipSuccess) return hip_fail(e, "projection launch");
    }
    return DASH_OK;
  } catch (...) {
    return fail(DASH_E_INVAL, "unexpected host exception");
  }
}

int dash_select_ragged(void* /*ctx*/, const dash_sel* p, const float* score, int n_total, int B, const int32_t* cu_n,
                       const int32_t* cu_k, int max_n, int k_total, int32_t* idx, void* stream) {
  try {
    if (!p) return fail(DASH_E_INVAL, "selection parameters are NULL");
    if (p->mode != DASH_SEL_TOPK) return fail(DASH_E_INVAL, "ragged selection supports top-k only");
    if (B < 1 || B > (1 << 20)) return fail(DASH_E_INVAL, "B %d out of range", B);
    if (max_n < 0 || max_n > (1 << 30)) return fail(DASH_E_INVAL, "max_n %d out of range", max_n);
    if (k_total < 0 || n_total < 0) return fail(DASH_E_INVAL, "n_total and k_total must be >= 0");
    if (max_n > n_total) return fail(DASH_E_INVAL, "max_n %d exceeds n_total %d", max_n, n_total);
    if (p->keep_first < 0 || p->keep_last < 0) return fail(DASH_E_INVAL, "forced counts must be >= 0");
    if (k_total == 0 || max_n == 0) return DASH_OK;
    if (!score || !idx || !cu_n || !cu_k) return fail(DASH_E_INVAL, "score, idx, cu_n and cu_k are required");
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int tr = trace_open(DASH_TR_SELECT, st);
    hipError_t e =
        dash::launch_topk_ragged(score, n_total, B, cu_n, cu_k, max_n, k_total, p->keep_first, p->keep_last, idx, st);
    trace_close(tr, st);
    if (e != hipSuccess) return hip_fail(e, "selection launch");
    return DASH_OK;
  } catch (...) {
    return fail(DASH_E_INVAL, "unexpected host exception");
  }
}

int dash_decode(void* /*ctx*/, const dash_shape* s, const void* Qd, int n_new, const void* Kc, const void* Vc,
                const int32_t* n_kv, void* Od, void* ws, size_t ws_bytes, void* stream) {
  try {
    int rc = check_shape(s, false);
    if (rc) return rc;
    if (s->dtype != DASH_BF16) return fail(DASH_E_DTYPE, "decode supports bf16 only");
    if (n_new < 1) return fail(DASH_E_INVAL, "n_new must be >= 1");
    if ((s->Hq / s->Hkv) * n_new > dash::decode_max_rows())
      return fail(DASH_E_SHAPE, "(Hq / Hkv) * n_new = %d exceeds %d", (s->Hq / s->Hkv) * n_new,
                  dash::decode_max_rows());
    rc = check_ptrs({{Qd, "Qd"}, {Kc, "Kc"}, {Vc, "Vc"}, {Od, "Od"}});
    if (rc) return rc;
    if (!n_kv) return fail(DASH_E_INVAL, "n_kv is NULL");
    const size_t need = align_up(dash::decode_workspace_bytes(s->B, s->S, s->Hkv, s->D));
    if (!ws || ws_bytes < need) return fail(DASH_E_WORKSPACE, "workspace needs %zu bytes, got %zu", need, ws ? ws_bytes : 0);
    if (!aligned16(ws)) return fail(DASH_E_ALIGN, "workspace is not 16-byte aligned");
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int tr = trace_open(DASH_TR_DECODE, st);
    hipError_t e = dash::launch_decode(s->D, Qd, Kc, Vc, n_kv, s->B, s->S, n_new, s->Hq, s->Hkv, Od,
                                       static_cast<float*>(ws), st);
    trace_close(tr, st);
    if (e != hipSuccess) return hip_fail(e, "decode launch");
    return DASH_OK;
  } catch (...) {
    return fail(DASH_E_INVAL, "unexpected host exception");
  }
}

int dash_score(void* /*ctx*/, const void* U, int dtype, int hidden, const int32_t* n_dev, int n_max, float* score,
               void* stream) {
  try {
    if (dtype != DASH_F32 && dtype != DASH_BF16) return fail(DASH_E_DTYPE, "dtype %d unsupported", dtype);
    if (n_max < 0) return fail(DASH_E_INVAL, "n_max must be >= 0");
    const int esz = dtype == DASH_BF16 ? 2 : 4;
    if (hidden < 1 || (static_cast<int64_t>(hidden) * esz) % 16 != 0)
      return fail(DASH_E_SHAPE, "hidden %d: rows must be a positive multiple of 16 bytes", hidden);
    if (static_cast<int64_t>(n_max) * hidden * esz / 16 >= (1ll << 31))
      return fail(DASH_E_SHAPE, "n_max * hidden too large");
    if (n_max == 0) return DASH_OK;
    int rc = check_ptrs({{U, "U"}});
    if (rc) return rc;
    if (!score) return fail(DASH_E_INVAL, "score is NULL");
    if (!aligned4(score)) return fail(DASH_E_ALIGN, "score is not 4-byte aligned");
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int tr = trace_open(DASH_TR_SCORE, st);
    hipError_t e = dash::launch_row_norm(dtype, U, n_dev, n_max, hidden, score, st);
    trace_close(tr, st);
    if (e != hipSuccess) return hip_fail(e, "score launch");
    return DASH_OK;
  } catch (...) {
    return fail(DASH_E_INVAL, "unexpected host exception");
  }
}

namespace {

int compact_many_impl(const int32_t* idx, const int32_t* n_dev, int n_max, const dash_gather* items, int count,
                      void* stream, int per_sample) {
  try {
    if (n_max < 0) return fail(DASH_E_INVAL, "n_max must be >= 0");
    if (count < 1 || count > dash::kMaxGather)
      return fail(DASH_E_INVAL, "count %d outside [1, %d]", count, dash::kMaxGather);
    if (!items) return fail(DASH_E_INVAL, "items is NULL");
    dash::GatherItem g[dash::kMaxGather];
    uint64_t chunks = 0;
    for (int j = 0; j < count; ++j) {
      const dash_gather& it = items[j];
      if (it.S < 0) return fail(DASH_E_INVAL, "items[%d].S must be >= 0", j);
      if (it.row_bytes == 0 || it.row_bytes % 16 != 0)
        return fail(DASH_E_ALIGN, "items[%d].row_bytes must be a positive multiple of 16", j);
      if (n_max > 0) {
        if (!it.X || !it.Xa) return fail(DASH_E_INVAL, "items[%d] has a NULL tensor", j);
        if (!aligned16(it.X) || !aligned16(it.Xa)) return fail(DASH_E_ALIGN, "items[%d] is not 16-byte aligned", j);
      }
      chunks += it.row_bytes / 16;
      g[j] = dash::GatherItem{it.X, it.S, it.row_bytes, it.Xa};
    }
    if (n_max == 0) return DASH_OK;
    if (!idx) return fail(DASH_E_INVAL, "idx is NULL");
    if (static_cast<uint64_t>(n_max) * chunks >= (1ull << 31))
      return fail(DASH_E_INVAL, "n_max * summed row_bytes too large");
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int tr = trace_open(DASH_TR_COMPACT, st);
    hipError_t e = dash::launch_compact_many(idx, n_dev, n_max, g, count, st, per_sample);
    trace_close(tr, st);
    if (e != hipSuccess) return hip_fail(e, "compaction launch");
    return DASH_OK;
  } catch (...) {
    return fail(DASH_E_INVAL, "unexpected host exception");
  }
}

}  // namespace

int dash_compact_many(void* /*ctx*/, const int32_t* idx, const int32_t* n_dev, int n_max, const dash_gather* items,
                      int count, void* stream) {
  return compact_many_impl(idx, n_dev, n_max, items, count, stream, 0);
}

int dash_compact_batch(void* /*ctx*/, const int32_t* idx, int B, int k, const dash_gather* items, int count,
                       void* stream) {
  if (B < 1 || k < 0) return fail(DASH_E_INVAL, "B must be >= 1 and k >= 0");
  if (static_cast<int64_t>(B) * k > (1ll << 30)) return fail(DASH_E_INVAL, "B * k too large");
  if (items && count >= 1 && count <= dash::kMaxGather)
    for (int j = 0; j < count; ++j)
      if (static_cast<int64_t>(B) * items[j].S > (1ll << 30))
        return fail(DASH_E_INVAL, "B * items[%d].S too large", j);
  return compact_many_impl(idx, nullptr, B * k, items, count, stream, k);
}

namespace {

// Post-halt attention (+ optional W_o GEMM and score) on n_max active rows.
// q_rows == nullptr: Q holds the compacted queries [B, n_max, Hq, D];
// otherwise Q is the full [B, S, Hq, D] and query r reads row q_rows[b, r].
int attn_active_impl(void* /*ctx*/, const dash_shape* s, const void* Qa, const int32_t* q_rows,
                     const int32_t* q_pos, const int32_t* n_dev, int n_max, const void* K, const void* V,
                     int kv_mode, void* Oa, const void* Wo, void* Ua, float* score, void* ws, size_t ws_bytes,
                     void* stream) {
  try {
    int rc = check_shape(s, false);
    if (rc) return rc;
    if (s->B > 1 && n_dev) return fail(DASH_E_SHAPE, "a device row count (n_dev) needs B == 1");
    if (kv_mode != DASH_KV_ACTIVE && kv_mode != DASH_KV_ALL) return fail(DASH_E_INVAL, "kv_mode %d unknown", kv_mode);
    if (n_max < 0 || n_max > s->S) return fail(DASH_E_INVAL, "n_max %d outside [0, S=%d]", n_max, s->S);
    if (n_max == 0) return DASH_OK;
    rc = check_ptrs({{Qa, q_rows ? "Q" : "Qa"}, {K, "K"}, {V, "V"}, {Oa, "Oa"}});
    if (rc) return rc;
    if (kv_mode == DASH_KV_ALL && !q_pos) return fail(DASH_E_INVAL, "kv_mode ALL needs q_pos");
    if (Wo) {
      rc = check_ptrs({{Wo, "Wo"}, {Ua, "Ua"}});
      if (rc) return rc;
      if (score) {
        if (!aligned16(score)) return fail(DASH_E_ALIGN, "score is not 16-byte aligned");
        const size_t need = score_ws_bytes(s, static_cast<int64_t>(s->B) * n_max);
        if (!ws || ws_bytes < need) return fail(DASH_E_WORKSPACE, "workspace needs %zu bytes, got %zu", need, ws ? ws_bytes : 0);
        if (!aligned16(ws)) return fail(DASH_E_ALIGN, "workspace is not 16-byte aligned");
      }
    } else if (Ua || score) {
      return fail(DASH_E_INVAL, "Ua / score need Wo");
    }
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int64_t qd = static_cast<int64_t>(s->Hq) * s->D;
    const int64_t kvd = static_cast<int64_t>(s->Hkv) * s->D;
    // ACTIVE: keys are the compacted rows aligned with the queries (their count
    // follows the query count, -1); ALL: the layer's S rows at their positions.
    const int n_kv = kv_mode == DASH_KV_ACTIVE ? (n_dev ? -1 : n_max) : s->S;
    const int32_t* qp = kv_mode == DASH_KV_ALL ? q_pos : nullptr;
    const int64_t kv_rows = kv_mode == DASH_KV_ACTIVE ? n_max : s->S;  // per sample
    int tr = trace_open(DASH_TR_ATTN_ACTIVE, st);
    dash::AttnBatch bt;
    bt.q_bs = (q_rows ? static_cast<int64_t>(s->S) : n_max) * qd;
    bt.kv_bs = kv_rows * kvd;
    bt.o_bs = n_max * qd;
    bt.qp_bs = n_max;
    bt.q_rows = q_rows;
    bt.q_rows_n = s->S;
    hipError_t e = dash::launch_attention(s->dtype, s->B, s->D, Qa, K, V, Oa, qp, n_dev, n_max, n_kv, s->Hq,
                                          s->Hkv, bt, st);
    trace_close(tr, st);
    if (e != hipSuccess) return hip_fail(e, "attention launch");
    if (Wo) {
      // the B samples' rows are contiguous: one GEMM over B * n_max rows
      tr = trace_open(DASH_TR_PROJ_ACTIVE, st);
      e = dash::launch_wo_gemm(s->dtype, Oa, Wo, Ua, score, static_cast<float*>(ws), n_dev, s->B * n_max,
                               s->hidden, static_cast<int>(qd), st);
      trace_close(tr, st);
      if (e != hipSuccess) return hip_fail(e, "projection launch");
    }
    return DASH_OK;
  } catch (...) {
    return fail(DASH_E_INVAL, "unexpected host exception");
  }
}

}  // namespace

int dash_attn_active(void* ctx, const dash_shape* s, const void* Qa, const int32_t* q_pos,
                     const int32_t* n_dev, int n_max, const void* K, const void* V, int kv_mode, void* Oa,
                     const void* Wo, void* Ua, float* score, void* ws, size_t ws_bytes, void* stream) {
  return attn_active_impl(ctx, s, Qa, nullptr, q_pos, n_dev, n_max, K, V, kv_mode, Oa, Wo, Ua, score, ws, ws_bytes,
                          stream);
}

int dash_attn_active_gather(void* ctx, const dash_shape* s, const void* Q, const int32_t* q_rows,
                            const int32_t* q_pos, const int32_t* n_dev, int n_max, const void* K, const void* V,
                            int kv_mode, void* Oa, const void* Wo, void* Ua, float* score, void* ws,
                            size_t ws_bytes, void* stream) {
  if (!q_rows) return fail(DASH_E_INVAL, "q_rows is NULL");
  return attn_active_impl(ctx, s, Q, q_rows, q_pos, n_dev, n_max, K, V, kv_mode, Oa, Wo, Ua, score, ws, ws_bytes,
                          stream);
}

}  // extern "C"
