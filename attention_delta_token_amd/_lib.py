"""ctypes binding of libdash.so (the C ABI in include/dash.h).

Argument marshalling only: tensors supply device pointers and shapes, torch's
current stream is passed through, and every step runs in the HIP library.
There is no fallback: if libdash.so is missing or a call fails, an exception
is raised.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, Structure, c_char_p, c_int, c_size_t, c_void_p

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdash.so")

DASH_OK, DASH_E_INVAL, DASH_E_SHAPE, DASH_E_DTYPE, DASH_E_ALIGN, DASH_E_WORKSPACE, DASH_E_HIP = range(7)
DASH_F32, DASH_BF16 = 0, 1
DASH_KV_ACTIVE, DASH_KV_ALL = 0, 1
DASH_SEL_TOPK, DASH_SEL_THRESHOLD, DASH_SEL_ORDER_STAT = 0, 1, 2
DASH_OP_ATTN_LAYER, DASH_OP_SELECT, DASH_OP_ATTN_ACTIVE, DASH_OP_DECODE = 0, 1, 2, 3

EXPORTED = ("dash_create", "dash_destroy", "dash_last_error", "dash_version", "dash_keep_count",
            "dash_percentile_rank", "dash_workspace_size",
            "dash_attn_layer", "dash_attn_layer_noalloc", "dash_select", "dash_compact", "dash_compact_many", "dash_compact_batch",
            "dash_attn_active", "dash_score", "dash_attn_layer_varlen", "dash_select_ragged",
            "dash_attn_active_varlen", "dash_attn_active_gather", "dash_decode",
            "dash_trace_start", "dash_trace_select", "dash_trace_stop", "dash_trace_read")
TRACE_OPS = ("attn_layer", "proj_layer", "attn_active", "proj_active", "select", "compact", "score", "decode")


class DashShape(Structure):
    _fields_ = [("B", c_int), ("S", c_int), ("Hq", c_int), ("Hkv", c_int), ("D", c_int), ("hidden", c_int),
                ("dtype", c_int)]


class DashGather(Structure):
    _fields_ = [("X", c_void_p), ("S", c_int), ("row_bytes", c_size_t), ("Xa", c_void_p)]


class DashSel(Structure):
    _fields_ = [("mode", c_int), ("k", c_int), ("rank", c_int), ("tau", c_void_p), ("patience", c_int),
                ("counters", c_void_p), ("keep_first", c_int), ("keep_last", c_int), ("n_counters", c_int)]


class DashError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"dash error {code}: {msg}")
        self.code = code


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libdash.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m attention_delta_token_amd.build`")
    lib = ctypes.CDLL(path)
    lib.dash_create.argtypes = [POINTER(c_void_p), c_int]
    lib.dash_create.restype = c_int
    lib.dash_destroy.argtypes = [c_void_p]
    lib.dash_destroy.restype = None
    lib.dash_last_error.argtypes = []
    lib.dash_last_error.restype = c_char_p
    lib.dash_version.argtypes = []
    lib.dash_version.restype = c_char_p
    lib.dash_keep_count.argtypes = [c_int, ctypes.c_double, c_int, c_int, POINTER(c_int)]
    lib.dash_keep_count.restype = c_int
    lib.dash_percentile_rank.argtypes = [c_int, c_int, POINTER(c_int)]
    lib.dash_percentile_rank.restype = c_int
    lib.dash_workspace_size.argtypes = [c_void_p, c_int, POINTER(DashShape), c_int]
    lib.dash_workspace_size.restype = c_size_t
    lib.dash_attn_layer.argtypes = [c_void_p, POINTER(DashShape), c_void_p, c_void_p, c_void_p, c_void_p,
                                    c_void_p, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]
    lib.dash_attn_layer.restype = c_int
    lib.dash_attn_layer_noalloc.argtypes = [c_void_p, POINTER(DashShape), c_void_p, c_void_p, c_void_p, c_void_p,
                                            c_void_p, c_void_p, c_void_p, c_void_p]
    lib.dash_attn_layer_noalloc.restype = c_int
    lib.dash_select.argtypes = [c_void_p, POINTER(DashSel), c_void_p, c_void_p, c_void_p, c_int, c_int,
                                c_void_p, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]
    lib.dash_select.restype = c_int
    lib.dash_compact.argtypes = [c_void_p, c_void_p, c_void_p, c_int, c_void_p, c_int, c_size_t, c_void_p,
                                 c_void_p]
    lib.dash_compact.restype = c_int
    lib.dash_compact_many.argtypes = [c_void_p, c_void_p, c_void_p, c_int, POINTER(DashGather), c_int, c_void_p]
    lib.dash_compact_many.restype = c_int
    lib.dash_compact_batch.argtypes = [c_void_p, c_void_p, c_int, c_int, POINTER(DashGather), c_int, c_void_p]
    lib.dash_compact_batch.restype = c_int
    lib.dash_score.argtypes = [c_void_p, c_void_p, c_int, c_int, c_void_p, c_int, c_void_p, c_void_p]
    lib.dash_score.restype = c_int
    lib.dash_attn_active.argtypes = [c_void_p, POINTER(DashShape), c_void_p, c_void_p, c_void_p, c_int,
                                     c_void_p, c_void_p, c_int, c_void_p, c_void_p, c_void_p, c_void_p,
                                     c_void_p, c_size_t, c_void_p]
    lib.dash_attn_active.restype = c_int
    lib.dash_attn_active_gather.argtypes = [c_void_p, POINTER(DashShape), c_void_p, c_void_p, c_void_p, c_void_p,
                                            c_int, c_void_p, c_void_p, c_int, c_void_p, c_void_p, c_void_p, c_void_p,
                                            c_void_p, c_size_t, c_void_p]
    lib.dash_attn_active_gather.restype = c_int
    lib.dash_attn_layer_varlen.argtypes = [c_void_p, POINTER(DashShape), c_void_p, c_int, c_void_p, c_void_p,
                                           c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t,
                                           c_void_p]
    lib.dash_attn_layer_varlen.restype = c_int
    lib.dash_select_ragged.argtypes = [c_void_p, POINTER(DashSel), c_void_p, c_int, c_int, c_void_p, c_void_p,
                                       c_int, c_int, c_void_p, c_void_p]
    lib.dash_select_ragged.restype = c_int
    lib.dash_attn_active_varlen.argtypes = [c_void_p, POINTER(DashShape), c_void_p, c_void_p, c_void_p, c_int,
                                            c_void_p, c_void_p, c_int, c_void_p, c_int, c_void_p, c_void_p,
                                            c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]
    lib.dash_attn_active_varlen.restype = c_int
    lib.dash_decode.argtypes = [c_void_p, POINTER(DashShape), c_void_p, c_int, c_void_p, c_void_p, c_void_p,
                                c_void_p, c_void_p, c_size_t, c_void_p]
    lib.dash_decode.restype = c_int
    lib.dash_trace_start.argtypes = [c_int]
    lib.dash_trace_start.restype = c_int
    lib.dash_trace_select.argtypes = [ctypes.c_uint]
    lib.dash_trace_select.restype = c_int
    lib.dash_trace_stop.argtypes = []
    lib.dash_trace_stop.restype = c_int
    lib.dash_trace_read.argtypes = [POINTER(c_int), POINTER(ctypes.c_float), c_int, POINTER(c_int)]
    lib.dash_trace_read.restype = c_int
    _lib = lib
    return lib


def _check(rc: int) -> None:
    if rc != DASH_OK:
        raise DashError(rc, load().dash_last_error().decode(errors="replace"))


def _ptr(t) -> int | None:
    """Device address of a tensor argument.  The kernels take dense row-major
    device memory, so a host tensor or a strided view is refused here rather
    than handed to a kernel (an int is taken as a raw device address)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError(f"tensor argument on {t.device}: the library takes device (cuda) tensors")
    if not t.is_contiguous():
        raise ValueError(f"tensor argument with strides {t.stride()} for shape {tuple(t.shape)}: "
                         "the library takes contiguous (row-major) tensors")
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _need(t, numel: int, dtype, name: str) -> None:
    """Check a tensor argument's element type and that it holds at least
    `numel` elements (the kernels write or read that many); None passes."""
    if t is None or isinstance(t, int):
        return
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if t.numel() < numel:
        raise ValueError(f"{name}: {t.numel()} elements, at least {numel} needed")


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return DASH_BF16
    if t.dtype == torch.float32:
        return DASH_F32
    raise DashError(DASH_E_DTYPE, f"unsupported tensor dtype {t.dtype}")


def make_shape(B: int, S: int, Hq: int, Hkv: int, D: int, hidden: int, dtype: int) -> DashShape:
    return DashShape(B, S, Hq, Hkv, D, hidden, dtype)


def version() -> str:
    return load().dash_version().decode()


def dash_workspace_size(op: int, shape: DashShape, n_max: int) -> int:
    return int(load().dash_workspace_size(None, op, ctypes.byref(shape), n_max))


def workspace(op: int, shape: DashShape, n_max: int, device="cuda") -> torch.Tensor:
    """Allocate (through torch) a workspace of dash_workspace_size bytes (at least 256)."""
    n = max(256, dash_workspace_size(op, shape, n_max))
    return torch.empty(n, dtype=torch.uint8, device=device)


def dash_attn_layer(Q, K, V, Wo, O, U, score=None, ws=None, stream=None) -> None:
    """Full-length layer: O = causal GQA attention, U = O·Wo^T, score = ||U_t||_2.

    Q [B,S,Hq,D] (or [S,Hq,D]); K, V [B,S,Hkv,D]; Wo [hidden, Hq*D]; O [B,S,Hq*D]; U [B,S,hidden]."""
    q = Q if Q.dim() == 4 else Q.unsqueeze(0)
    k = K if K.dim() == 4 else K.unsqueeze(0)
    B, S, Hq, D = q.shape
    Hkv, hidden = k.shape[2], Wo.shape[0]
    for t, n, name in ((K, B * S * Hkv * D, "K"), (V, B * S * Hkv * D, "V"), (Wo, hidden * Hq * D, "Wo"),
                       (O, B * S * Hq * D, "O"), (U, B * S * hidden, "U")):
        _need(t, n, Q.dtype, name)
    _need(score, B * S, torch.float32, "score")
    shape = make_shape(B, S, Hq, Hkv, D, hidden, _dtype_code(Q))
    _check(load().dash_attn_layer(None, ctypes.byref(shape), _ptr(Q), _ptr(K), _ptr(V), _ptr(Wo), _ptr(O),
                                  _ptr(U), _ptr(score), _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(),
                                  _stream(stream)))


def dash_attn_layer_noalloc(Q, K, V, Wo, O, U, score=None, stream=None) -> None:
    """dash_attn_layer without a workspace: the score's partial sums live in the
    library's built-in per-GPU scratch (see include/dash.h for its limit)."""
    q = Q if Q.dim() == 4 else Q.unsqueeze(0)
    k = K if K.dim() == 4 else K.unsqueeze(0)
    B, S, Hq, D = q.shape
    Hkv, hidden = k.shape[2], Wo.shape[0]
    for t, n, name in ((K, B * S * Hkv * D, "K"), (V, B * S * Hkv * D, "V"), (Wo, hidden * Hq * D, "Wo"),
                       (O, B * S * Hq * D, "O"), (U, B * S * hidden, "U")):
        _need(t, n, Q.dtype, name)
    _need(score, B * S, torch.float32, "score")
    shape = make_shape(B, S, Hq, Hkv, D, hidden, _dtype_code(Q))
    _check(load().dash_attn_layer_noalloc(None, ctypes.byref(shape), _ptr(Q), _ptr(K), _ptr(V), _ptr(Wo), _ptr(O),
                                          _ptr(U), _ptr(score), _stream(stream)))


def dash_select(score, idx=None, *, mode: int = DASH_SEL_TOPK, k: int = 0, rank: int = 0, tau=None,
                patience: int = 2, counters=None, pos=None, n_dev=None, n_max: int | None = None, rows: int = 1,
                n_out=None, tau_out=None, keep_first: int = 0, keep_last: int = 0, status=None,
                stream=None) -> None:
    """Top-k / order statistic / threshold step (see include/dash.h).  For top-k
    with forced retention, k is the total kept count (see keep_count).
    status: optional int32 device tensor of at least `rows` entries that
    receives each row's number of NaN scores (the call's workspace)."""
    if n_max is None:
        n_max = score.shape[-1] if score is not None else 0
    _need(score, rows * n_max, torch.float32, "score")
    _need(idx, rows * k if mode == DASH_SEL_TOPK else (n_max if mode == DASH_SEL_THRESHOLD else 0), torch.int32,
          "idx")
    _need(pos, n_max if mode != DASH_SEL_ORDER_STAT else 0, torch.int32, "pos")
    _need(counters, 0, torch.uint8, "counters")
    _need(n_dev, 1, torch.int32, "n_dev")
    _need(n_out, 1, torch.int32, "n_out")
    _need(tau, 1, torch.float32, "tau")
    _need(tau_out, 1, torch.float32, "tau_out")
    _need(status, rows, torch.int32, "status")
    n_counters = counters.numel() if counters is not None else 0
    sel = DashSel(mode, k, rank, _ptr(tau), patience, _ptr(counters), keep_first, keep_last, n_counters)
    ws_bytes = status.numel() * status.element_size() if status is not None else 0
    _check(load().dash_select(None, ctypes.byref(sel), _ptr(score), _ptr(pos), _ptr(n_dev), n_max, rows,
                              _ptr(idx), _ptr(n_out), _ptr(tau_out), _ptr(status), ws_bytes, _stream(stream)))


def select_status(rows: int = 1, device="cuda", n_max: int = 0) -> torch.Tensor:
    """An int32 device buffer for dash_select's NaN counts (one word per row);
    with n_max, also the scratch a single long row's top-k spreads over many
    workgroups with (dash_workspace_size(DASH_OP_SELECT, ..., n_max))."""
    n = dash_workspace_size(DASH_OP_SELECT, make_shape(rows, 1, 1, 1, 1, 1, DASH_F32), n_max)
    return torch.zeros(max(n, 256) // 4, dtype=torch.int32, device=device)


def keep_count(T: int, keep: float, keep_first: int = 0, keep_last: int = 0) -> int:
    """Kept count of the one-shot policy, K_eff (dash_keep_count)."""
    out = c_int(0)
    _check(load().dash_keep_count(T, float(keep), keep_first, keep_last, ctypes.byref(out)))
    return out.value


def percentile_rank(n: int, pct: int) -> int:
    """Rank of the nearest-rank pct-th percentile among n scores (dash_percentile_rank)."""
    out = c_int(0)
    _check(load().dash_percentile_rank(n, pct, ctypes.byref(out)))
    return out.value


def dash_compact(idx, X, Xa, n_dev=None, n_max: int | None = None, stream=None) -> None:
    """Xa[r] = X[idx[r]] for r < n (n = *n_dev or n_max); X is [S, ...] row-major."""
    S = X.shape[0]
    row_bytes = X[0].numel() * X.element_size() if S > 0 else Xa[0].numel() * Xa.element_size()
    if n_max is None:
        n_max = idx.shape[0]
    _need(idx, n_max, torch.int32, "idx")
    _need(Xa, n_max * row_bytes // X.element_size(), X.dtype, "Xa")
    _check(load().dash_compact(None, _ptr(idx), _ptr(n_dev), n_max, _ptr(X), S, row_bytes, _ptr(Xa),
                               _stream(stream)))


def dash_compact_many(idx, pairs, n_dev=None, n_max: int | None = None, stream=None) -> None:
    """One launch gathering several tensors at the same rows: for each (X, Xa)
    in pairs, Xa[r] = X[idx[r]] for r < n (at most 4 pairs)."""
    if n_max is None:
        n_max = idx.shape[0]
    _need(idx, n_max, torch.int32, "idx")
    arr = (DashGather * len(pairs))()
    for j, (X, Xa) in enumerate(pairs):
        S = X.shape[0]
        row_bytes = X[0].numel() * X.element_size() if S > 0 else Xa[0].numel() * Xa.element_size()
        _need(Xa, n_max * row_bytes // X.element_size(), X.dtype, f"pairs[{j}] Xa")
        arr[j] = DashGather(_ptr(X), S, row_bytes, _ptr(Xa))
    _check(load().dash_compact_many(None, _ptr(idx), _ptr(n_dev), n_max, arr, len(pairs), _stream(stream)))


def dash_compact_batch(idx, pairs, stream=None) -> None:
    """Per-sample gathers of B samples in one launch: idx [B, k] local positions;
    for each (X [B, S, ...], Xa [B, k, ...]) in pairs, Xa[b, r] = X[b, idx[b, r]]."""
    B, k = idx.shape
    _need(idx, 0, torch.int32, "idx")
    arr = (DashGather * len(pairs))()
    for j, (X, Xa) in enumerate(pairs):
        S = X.shape[1]
        row_bytes = X[0, 0].numel() * X.element_size() if S > 0 else Xa[0, 0].numel() * Xa.element_size()
        _need(Xa, B * k * row_bytes // X.element_size(), X.dtype, f"pairs[{j}] Xa")
        arr[j] = DashGather(_ptr(X), S, row_bytes, _ptr(Xa))
    _check(load().dash_compact_batch(None, _ptr(idx), B, k, arr, len(pairs), _stream(stream)))


def dash_score(U, score, n_dev=None, n_max: int | None = None, stream=None) -> None:
    """score[t] = ||U[t]||_2 for t < n (U [n_max, hidden], bf16 or fp32)."""
    if n_max is None:
        n_max = U.shape[0]
    hidden = U[0].numel() if U.shape[0] > 0 else U.shape[-1]
    _need(score, n_max, torch.float32, "score")
    _check(load().dash_score(None, _ptr(U), _dtype_code(U), hidden, _ptr(n_dev), n_max, _ptr(score),
                             _stream(stream)))


def dash_attn_active(Qa, K, V, kv_mode: int, Oa, q_pos=None, n_dev=None, n_max: int | None = None, Wo=None,
                     Ua=None, score=None, ws=None, S: int | None = None, hidden: int | None = None,
                     stream=None) -> None:
    """Post-halt attention (see include/dash.h).  Qa [n,Hq,D] or [B,n,Hq,D];
    K, V [n or S, Hkv, D] or [B, n or S, Hkv, D]."""
    if Qa.dim() == 4:
        B, n_cap, Hq, D = Qa.shape
        kv_rows, Hkv = K.shape[1], K.shape[2]
    else:
        B = 1
        n_cap, Hq, D = Qa.shape
        kv_rows, Hkv = K.shape[0], K.shape[1]
    if n_max is None:
        n_max = n_cap
    if S is None:
        S = kv_rows if kv_mode == DASH_KV_ALL else n_max
    if hidden is None:
        hidden = Wo.shape[0] if Wo is not None else Hq * D
    _need(V, K.numel(), Qa.dtype, "V")
    _need(K, 0, Qa.dtype, "K")
    _need(Oa, B * n_max * Hq * D, Qa.dtype, "Oa")
    _need(Wo, hidden * Hq * D, Qa.dtype, "Wo")
    _need(Ua, B * n_max * hidden, Qa.dtype, "Ua")
    _need(score, B * n_max, torch.float32, "score")
    _need(q_pos, B * n_max, torch.int32, "q_pos")
    _need(n_dev, 1, torch.int32, "n_dev")
    shape = make_shape(B, S, Hq, Hkv, D, hidden, _dtype_code(Qa))
    _check(load().dash_attn_active(None, ctypes.byref(shape), _ptr(Qa), _ptr(q_pos), _ptr(n_dev), n_max, _ptr(K),
                                   _ptr(V), kv_mode, _ptr(Oa), _ptr(Wo), _ptr(Ua), _ptr(score), _ptr(ws),
                                   0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def dash_attn_active_gather(Q, q_rows, K, V, kv_mode: int, Oa, q_pos=None, n_dev=None, n_max: int | None = None,
                            Wo=None, Ua=None, score=None, ws=None, hidden: int | None = None,
                            stream=None) -> None:
    """Post-halt attention reading its queries from the full-length Q through
    q_rows (see include/dash.h).  Q [S,Hq,D] or [B,S,Hq,D]; q_rows [n] or
    [B, n] (device int32); K, V [n or S, Hkv, D] (or with a leading B)."""
    if Q.dim() == 4:
        B, S, Hq, D = Q.shape
        Hkv = K.shape[2]
    else:
        B = 1
        S, Hq, D = Q.shape
        Hkv = K.shape[1]
    n_cap = q_rows.shape[-1]
    if n_max is None:
        n_max = n_cap
    if hidden is None:
        hidden = Wo.shape[0] if Wo is not None else Hq * D
    _need(q_rows, B * n_max, torch.int32, "q_rows")
    kv_rows = S if kv_mode == DASH_KV_ALL else n_max
    _need(K, B * kv_rows * Hkv * D, Q.dtype, "K")
    _need(V, B * kv_rows * Hkv * D, Q.dtype, "V")
    _need(Oa, B * n_max * Hq * D, Q.dtype, "Oa")
    _need(Wo, hidden * Hq * D, Q.dtype, "Wo")
    _need(Ua, B * n_max * hidden, Q.dtype, "Ua")
    _need(score, B * n_max, torch.float32, "score")
    _need(q_pos, B * n_max, torch.int32, "q_pos")
    _need(n_dev, 1, torch.int32, "n_dev")
    shape = make_shape(B, S, Hq, Hkv, D, hidden, _dtype_code(Q))
    _check(load().dash_attn_active_gather(None, ctypes.byref(shape), _ptr(Q), _ptr(q_rows), _ptr(q_pos),
                                          _ptr(n_dev), n_max, _ptr(K), _ptr(V), kv_mode, _ptr(Oa), _ptr(Wo),
                                          _ptr(Ua), _ptr(score), _ptr(ws),
                                          0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def dash_attn_layer_varlen(Q, K, V, Wo, O, U, cu_seqlens, max_len: int, score=None, ws=None, stream=None) -> None:
    """Packed batch: Q [T, Hq, D], K, V [T, Hkv, D], cu_seqlens [B+1] (device int32), max_len = longest sample."""
    T, Hq, D = Q.shape
    B = cu_seqlens.shape[0] - 1
    Hkv, hidden = K.shape[1], Wo.shape[0]
    for t, n, name in ((K, T * Hkv * D, "K"), (V, T * Hkv * D, "V"), (Wo, hidden * Hq * D, "Wo"),
                       (O, T * Hq * D, "O"), (U, T * hidden, "U")):
        _need(t, n, Q.dtype, name)
    _need(score, T, torch.float32, "score")
    _need(cu_seqlens, B + 1, torch.int32, "cu_seqlens")
    shape = make_shape(B, max_len, Hq, Hkv, D, hidden, _dtype_code(Q))
    _check(load().dash_attn_layer_varlen(None, ctypes.byref(shape), _ptr(cu_seqlens), T, _ptr(Q), _ptr(K), _ptr(V),
                                         _ptr(Wo), _ptr(O), _ptr(U), _ptr(score), _ptr(ws),
                                         0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def dash_select_ragged(score, idx, cu_n, cu_k, max_n: int, keep_first: int = 0, keep_last: int = 0,
                       stream=None) -> None:
    """Per-sample top-k of a packed score vector; idx receives packed row indices."""
    sel = DashSel(DASH_SEL_TOPK, 0, 0, None, 2, None, keep_first, keep_last)
    B = cu_n.shape[0] - 1
    _need(score, 0, torch.float32, "score")
    _need(idx, 0, torch.int32, "idx")
    _need(cu_n, B + 1, torch.int32, "cu_n")
    _need(cu_k, B + 1, torch.int32, "cu_k")
    _check(load().dash_select_ragged(None, ctypes.byref(sel), _ptr(score), score.shape[0], B, _ptr(cu_n), _ptr(cu_k),
                                     max_n, idx.shape[0], _ptr(idx), _stream(stream)))


def dash_attn_active_varlen(Qa, K, V, kv_mode: int, Oa, cu_q, max_rows: int, q_pos=None, cu_kv=None, Wo=None,
                            Ua=None, score=None, ws=None, stream=None) -> None:
    """Packed post-halt attention: Qa [n_total, Hq, D]; K, V [n_total or kv_total, Hkv, D]."""
    n_total, Hq, D = Qa.shape
    B = cu_q.shape[0] - 1
    hidden = Wo.shape[0] if Wo is not None else Hq * D
    _need(V, K.numel(), Qa.dtype, "V")
    _need(Oa, n_total * Hq * D, Qa.dtype, "Oa")
    _need(Wo, hidden * Hq * D, Qa.dtype, "Wo")
    _need(Ua, n_total * hidden, Qa.dtype, "Ua")
    _need(score, n_total, torch.float32, "score")
    _need(q_pos, n_total, torch.int32, "q_pos")
    _need(cu_q, B + 1, torch.int32, "cu_q")
    _need(cu_kv, B + 1, torch.int32, "cu_kv")
    shape = make_shape(B, max_rows, Hq, K.shape[1], D, hidden, _dtype_code(Qa))
    _check(load().dash_attn_active_varlen(None, ctypes.byref(shape), _ptr(Qa), _ptr(q_pos), _ptr(cu_q), n_total,
                                          _ptr(K), _ptr(V), kv_mode, _ptr(cu_kv), K.shape[0], _ptr(Oa), _ptr(Wo),
                                          _ptr(Ua), _ptr(score), _ptr(ws),
                                          0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def dash_decode(Qd, Kc, Vc, n_kv, Od, ws=None, stream=None) -> None:
    """Decode attention: Qd [B, n_new, Hq, D]; Kc, Vc [B, S, Hkv, D] caches with n_kv [B] (device) rows."""
    B, n_new, Hq, D = Qd.shape
    S, Hkv = Kc.shape[1], Kc.shape[2]
    _need(Kc, B * S * Hkv * D, Qd.dtype, "Kc")
    _need(Vc, B * S * Hkv * D, Qd.dtype, "Vc")
    _need(Od, B * n_new * Hq * D, Qd.dtype, "Od")
    _need(n_kv, B, torch.int32, "n_kv")
    shape = make_shape(B, S, Hq, Hkv, D, Hq * D, _dtype_code(Qd))
    if ws is None:
        ws = workspace(DASH_OP_DECODE, shape, n_new, device=Qd.device)
    _check(load().dash_decode(None, ctypes.byref(shape), _ptr(Qd), n_new, _ptr(Kc), _ptr(Vc), _ptr(n_kv), _ptr(Od),
                              _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def trace_start(capacity: int) -> None:
    """Start bracketing every library launch with HIP events (measurement only)."""
    _check(load().dash_trace_start(capacity))


def trace_select(ops) -> None:
    """Record only these launch-group kinds (names from TRACE_OPS) from now on."""
    mask = 0
    for name in ops:
        mask |= 1 << TRACE_OPS.index(name)
    _check(load().dash_trace_select(ctypes.c_uint(mask)))


def trace_stop() -> None:
    _check(load().dash_trace_stop())


def trace_read(max_records: int = 1 << 16) -> list[tuple[str, float]]:
    """Wait for the recorded events; return [(op name, milliseconds)] in launch order."""
    ops = (c_int * max_records)()
    ms = (ctypes.c_float * max_records)()
    n = c_int(0)
    _check(load().dash_trace_read(ops, ms, max_records, ctypes.byref(n)))
    return [(TRACE_OPS[ops[i]], float(ms[i])) for i in range(n.value)]
