"""The C-ABI library loads, exports every symbol include/dash.h declares, and
rejects invalid arguments before touching the GPU.  CPU only: no call here
reaches a kernel launch."""
import ctypes
import os
import re

import pytest

import attention_delta_token_amd as dash
from attention_delta_token_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dash.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(dash.LIB_PATH):
        pytest.fail("libdash.so is not built (run __graft_entry__.build())")
    return dash.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dash_[a-z_]+)\s*\(", text)))


def test_header_declares_the_four_calls():
    names = declared_functions()
    for n in ("dash_attn_layer", "dash_select", "dash_compact", "dash_attn_active"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(L.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n


def test_version(lib):
    assert "gfx950" in dash.version()


def _shape(**kw):
    d = dict(B=1, S=64, Hq=4, Hkv=2, D=128, hidden=512, dtype=L.DASH_BF16)
    d.update(kw)
    return L.DashShape(d["B"], d["S"], d["Hq"], d["Hkv"], d["D"], d["hidden"], d["dtype"])


def _last(lib):
    return lib.dash_last_error().decode()


FAKE = 0x10000  # aligned, never dereferenced: validation fails before any launch


def test_attn_layer_validation(lib):
    f = lib.dash_attn_layer
    p = [FAKE] * 6
    assert f(None, None, *p, None, None, 0, None) == L.DASH_E_INVAL
    assert f(None, ctypes.byref(_shape(Hq=6, Hkv=4)), *p, None, None, 0, None) == L.DASH_E_SHAPE
    assert "multiple" in _last(lib)
    assert f(None, ctypes.byref(_shape(D=96)), *p, None, None, 0, None) == L.DASH_E_SHAPE
    assert f(None, ctypes.byref(_shape(dtype=7)), *p, None, None, 0, None) == L.DASH_E_DTYPE
    assert f(None, ctypes.byref(_shape(S=0)), *p, None, None, 0, None) == L.DASH_E_SHAPE
    assert f(None, ctypes.byref(_shape()), None, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, 0, None) == L.DASH_E_INVAL
    assert "Q is NULL" in _last(lib)
    assert f(None, ctypes.byref(_shape()), FAKE + 4, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, 0, None) == L.DASH_E_ALIGN
    # score requested with a missing or short workspace
    assert f(None, ctypes.byref(_shape()), *p, FAKE, None, 0, None) == L.DASH_E_WORKSPACE
    need = lib.dash_workspace_size(None, L.DASH_OP_ATTN_LAYER, ctypes.byref(_shape()), 64)
    assert need >= 64 * 4  # at least one fp32 partial per row
    assert f(None, ctypes.byref(_shape()), *p, FAKE, FAKE, need - 1, None) == L.DASH_E_WORKSPACE


def _sel(mode, k=0, rank=0, tau=None, patience=2, counters=None, f=0, l=0, n_counters=0):
    return L.DashSel(mode, k, rank, tau, patience, counters, f, l, n_counters)


def test_select_validation(lib):
    """Every case here fails validation (or has nothing to do), so no kernel is
    launched on the placeholder pointers."""
    f = lib.dash_select
    sel = _sel(L.DASH_SEL_TOPK, k=5)
    assert f(None, None, FAKE, None, None, 10, 1, FAKE, None, None, None, 0, None) == L.DASH_E_INVAL
    assert f(None, ctypes.byref(sel), FAKE, None, None, 4, 1, FAKE, None, None, None, 0, None) == L.DASH_E_INVAL
    assert "outside" in _last(lib)
    # a device count (or a kept-count output) with several rows
    assert f(None, ctypes.byref(sel), FAKE, None, FAKE, 10, 2, FAKE, None, None, None, 0, None) == L.DASH_E_INVAL
    assert "single row" in _last(lib)
    assert f(None, ctypes.byref(sel), FAKE, None, None, 10, 2, FAKE, FAKE, None, None, 0, None) == L.DASH_E_INVAL
    assert f(None, ctypes.byref(sel), FAKE, FAKE, None, 10, 2, FAKE, None, None, None, 0, None) == L.DASH_E_INVAL
    assert f(None, ctypes.byref(sel), None, None, None, 10, 1, FAKE, None, None, None, 0, None) == L.DASH_E_INVAL
    sel0 = _sel(L.DASH_SEL_TOPK)
    assert f(None, ctypes.byref(sel0), None, None, None, 10, 1, None, None, None, None, 0, None) == L.DASH_OK
    # the NaN status needs 4 bytes per row of workspace (256 at least)
    assert f(None, ctypes.byref(sel), FAKE, None, None, 10, 1, FAKE, None, None, FAKE, 255, None) == \
        L.DASH_E_WORKSPACE
    assert f(None, ctypes.byref(sel), FAKE, None, None, 10, 100, FAKE, None, None, FAKE, 256, None) == \
        L.DASH_E_WORKSPACE
    assert f(None, ctypes.byref(sel), FAKE, None, None, 10, 1, FAKE, None, None, FAKE + 2, 256, None) == \
        L.DASH_E_ALIGN
    forced = _sel(L.DASH_SEL_TOPK, k=5, f=64)
    assert f(None, ctypes.byref(forced), FAKE, None, None, 10, 1, FAKE, None, None, None, 0, None) == L.DASH_E_INVAL
    # forced retention: f + l must not exceed k; negative counts rejected; top-k only
    for kf, kl in ((3, 3), (-1, 0), (0, -2)):
        bad_f = _sel(L.DASH_SEL_TOPK, k=5, f=kf, l=kl)
        assert f(None, ctypes.byref(bad_f), FAKE, None, None, 10, 1, FAKE, None, None, None, 0, None) == L.DASH_E_INVAL
    assert "keep_first" in _last(lib)
    os_f = _sel(L.DASH_SEL_ORDER_STAT, rank=3, f=1)
    assert f(None, ctypes.byref(os_f), FAKE, None, None, 10, 1, None, None, FAKE, None, 0, None) == L.DASH_E_INVAL
    assert "top-k only" in _last(lib)
    os_ = _sel(L.DASH_SEL_ORDER_STAT, rank=11)
    assert f(None, ctypes.byref(os_), FAKE, None, None, 10, 1, None, None, FAKE, None, 0, None) == L.DASH_E_INVAL
    th = _sel(L.DASH_SEL_THRESHOLD, tau=FAKE, patience=0, counters=FAKE, n_counters=10)
    assert f(None, ctypes.byref(th), FAKE, None, None, 10, 1, FAKE, FAKE, None, None, 0, None) == L.DASH_E_INVAL
    assert "patience" in _last(lib)
    th = _sel(L.DASH_SEL_THRESHOLD, tau=FAKE, counters=FAKE, n_counters=0)
    assert f(None, ctypes.byref(th), FAKE, None, None, 10, 1, FAKE, FAKE, None, None, 0, None) == L.DASH_E_INVAL
    assert "n_counters" in _last(lib)
    th = _sel(L.DASH_SEL_THRESHOLD, tau=FAKE, counters=FAKE, n_counters=9)  # rows are positions 0..9
    assert f(None, ctypes.byref(th), FAKE, None, None, 10, 1, FAKE, FAKE, None, None, 0, None) == L.DASH_E_INVAL
    assert "n_counters" in _last(lib)
    th = _sel(L.DASH_SEL_THRESHOLD, tau=FAKE, counters=FAKE, n_counters=10)
    assert f(None, ctypes.byref(th), FAKE, FAKE, None, 10, 1, FAKE, FAKE, None, None, 0, None) == L.DASH_E_INVAL
    assert "alias" in _last(lib)
    bad = _sel(9)
    assert f(None, ctypes.byref(bad), FAKE, None, None, 10, 1, FAKE, None, None, None, 0, None) == L.DASH_E_INVAL


def test_keep_count_matches_the_oracle(lib, golden_dir):
    """dash_keep_count / dash_percentile_rank against the hand-worked counts and
    the oracle's K_eff (which the fixtures pin)."""
    import json
    import oracle
    c = json.load(open(os.path.join(golden_dir, "counts.json")))
    for e in c["keep"]:
        assert dash.keep_count(e["S"], e["keep"]) == e["k"]
    for e in c["rank"]:
        assert dash.percentile_rank(e["S"], e["pct"]) == e["r"]
    for e in c.get("forced", []):
        assert dash.keep_count(e["T"], e["keep"], e["f"], e["l"]) == e["k"]
    for T in (0, 1, 7, 96, 97, 512, 8192, 131072):
        for keep in (0.0, 0.3, 0.333, 0.5, 0.667, 1.0):
            for fl in ((0, 0), (64, 32), (1, 0), (0, 1)):
                if sum(fl) <= T:
                    assert dash.keep_count(T, keep, *fl) == oracle.effective_keep_count(T, keep, *fl)
        if T >= 1:
            for pct in (0, 1, 30, 50, 99, 100):
                assert dash.percentile_rank(T, pct) == oracle.percentile_rank(T, pct)
    out = ctypes.c_int(-5)
    assert lib.dash_keep_count(10, 1.5, 0, 0, ctypes.byref(out)) == L.DASH_E_INVAL and out.value == -5
    assert lib.dash_keep_count(10, 0.5, 6, 5, ctypes.byref(out)) == L.DASH_E_INVAL
    assert lib.dash_keep_count(-1, 0.5, 0, 0, ctypes.byref(out)) == L.DASH_E_INVAL
    assert lib.dash_keep_count(10, float("nan"), 0, 0, ctypes.byref(out)) == L.DASH_E_INVAL
    assert lib.dash_keep_count(10, 0.5, 0, 0, None) == L.DASH_E_INVAL
    assert lib.dash_percentile_rank(0, 30, ctypes.byref(out)) == L.DASH_E_INVAL
    assert lib.dash_percentile_rank(10, 101, ctypes.byref(out)) == L.DASH_E_INVAL


def test_kv_extent_limit(lib):
    """One sample's K must stay below 4 GiB (32-bit buffer offsets in the
    attention kernel): S * Hkv * D * 2 = 2^32 is refused, one row less passes the
    shape check (and then fails on the NULL pointers)."""
    f = lib.dash_attn_layer
    big = _shape(S=1 << 21, Hq=8, Hkv=8, D=128, hidden=1024)
    assert f(None, ctypes.byref(big), *([FAKE] * 6), None, None, 0, None) == L.DASH_E_SHAPE
    assert "4 GiB" in _last(lib)
    ok = _shape(S=(1 << 21) - 1, Hq=8, Hkv=8, D=128, hidden=1024)
    assert f(None, ctypes.byref(ok), None, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, 0, None) == L.DASH_E_INVAL
    f32 = _shape(S=1 << 20, Hq=8, Hkv=8, D=128, hidden=1024, dtype=L.DASH_F32)
    assert f(None, ctypes.byref(f32), *([FAKE] * 6), None, None, 0, None) == L.DASH_E_SHAPE


def test_compact_validation(lib):
    f = lib.dash_compact
    assert f(None, FAKE, None, 10, FAKE, 10, 24, FAKE, None) == L.DASH_E_ALIGN
    assert f(None, FAKE, None, 10, FAKE, 10, 0, FAKE, None) == L.DASH_E_ALIGN
    assert f(None, None, None, 10, FAKE, 10, 32, FAKE, None) == L.DASH_E_INVAL
    assert f(None, FAKE, None, -1, FAKE, 10, 32, FAKE, None) == L.DASH_E_INVAL
    assert f(None, FAKE, None, 10, FAKE + 8, 10, 32, FAKE, None) == L.DASH_E_ALIGN
    assert f(None, FAKE, None, 0, None, 10, 32, None, None) == L.DASH_OK  # nothing to do


def test_compact_many_validation(lib):
    f = lib.dash_compact_many
    G = L.DashGather

    def arr(*items):
        a = (G * len(items))()
        for j, it in enumerate(items):
            a[j] = G(*it)
        return a
    good = (FAKE, 10, 32, FAKE)
    assert f(None, FAKE, None, 10, arr(good), 0, None) == L.DASH_E_INVAL
    assert f(None, FAKE, None, 10, arr(good, good, good, good, good), 5, None) == L.DASH_E_INVAL
    assert f(None, FAKE, None, 10, None, 1, None) == L.DASH_E_INVAL
    assert f(None, FAKE, None, 10, arr(good, (FAKE, 10, 24, FAKE)), 2, None) == L.DASH_E_ALIGN
    assert f(None, FAKE, None, 10, arr(good, (FAKE + 8, 10, 32, FAKE)), 2, None) == L.DASH_E_ALIGN
    assert f(None, FAKE, None, 10, arr((None, 10, 32, FAKE)), 1, None) == L.DASH_E_INVAL
    assert f(None, FAKE, None, 10, arr((FAKE, -1, 32, FAKE)), 1, None) == L.DASH_E_INVAL
    assert f(None, None, None, 10, arr(good), 1, None) == L.DASH_E_INVAL
    assert f(None, FAKE, None, 1 << 20, arr((FAKE, 10, 1 << 20, FAKE)), 1, None) == L.DASH_E_INVAL
    assert f(None, None, None, 0, arr(good), 1, None) == L.DASH_OK  # nothing to do


def test_score_validation(lib):
    f = lib.dash_score
    assert f(None, FAKE, 7, 256, None, 10, FAKE, None) == L.DASH_E_DTYPE
    assert f(None, FAKE, L.DASH_BF16, 12, None, 10, FAKE, None) == L.DASH_E_SHAPE  # 24-byte rows
    assert f(None, FAKE, L.DASH_F32, 0, None, 10, FAKE, None) == L.DASH_E_SHAPE
    assert f(None, FAKE + 8, L.DASH_BF16, 256, None, 10, FAKE, None) == L.DASH_E_ALIGN
    assert f(None, FAKE, L.DASH_BF16, 256, None, 10, None, None) == L.DASH_E_INVAL
    assert f(None, FAKE, L.DASH_BF16, 256, None, 10, FAKE + 2, None) == L.DASH_E_ALIGN
    assert f(None, None, L.DASH_BF16, 256, None, 0, None, None) == L.DASH_OK  # nothing to do


def test_compact_batch_validation(lib):
    f = lib.dash_compact_batch
    G = L.DashGather
    one = (G * 1)(G(FAKE, 10, 32, FAKE))
    assert f(None, FAKE, 0, 4, one, 1, None) == L.DASH_E_INVAL
    assert f(None, FAKE, 2, -1, one, 1, None) == L.DASH_E_INVAL
    assert f(None, FAKE, 2, 4, one, 0, None) == L.DASH_E_INVAL
    bad = (G * 1)(G(FAKE, 10, 40, FAKE))
    assert f(None, FAKE, 2, 4, bad, 1, None) == L.DASH_E_ALIGN
    assert f(None, None, 2, 4, one, 1, None) == L.DASH_E_INVAL
    assert f(None, None, 2, 0, one, 1, None) == L.DASH_OK  # nothing to do


def test_ragged_validation(lib):
    s = _shape(B=3, S=64)
    f = lib.dash_attn_layer_varlen
    ptrs = [FAKE] * 6
    assert f(None, ctypes.byref(s), FAKE, 3 * 64 + 1, *ptrs, None, None, 0, None) == L.DASH_E_SHAPE
    assert f(None, ctypes.byref(s), None, 100, *ptrs, None, None, 0, None) == L.DASH_E_INVAL
    assert f(None, ctypes.byref(s), FAKE, 100, *ptrs, FAKE, None, 0, None) == L.DASH_E_WORKSPACE
    assert f(None, ctypes.byref(s), FAKE, 0, *ptrs, None, None, 0, None) == L.DASH_OK
    g = lib.dash_select_ragged
    top = _sel(L.DASH_SEL_TOPK)
    assert g(None, ctypes.byref(_sel(L.DASH_SEL_ORDER_STAT, rank=1)), FAKE, 10, 2, FAKE,
             FAKE, 8, 5, FAKE, None) == L.DASH_E_INVAL
    assert g(None, ctypes.byref(top), FAKE, 10, 2, FAKE, FAKE, 11, 5, FAKE, None) == L.DASH_E_INVAL  # max_n > n_total
    assert g(None, ctypes.byref(top), FAKE, 10, 2, None, FAKE, 8, 5, FAKE, None) == L.DASH_E_INVAL
    assert g(None, ctypes.byref(top), FAKE, 10, 0, FAKE, FAKE, 8, 5, FAKE, None) == L.DASH_E_INVAL
    assert g(None, ctypes.byref(top), None, 10, 2, None, None, 8, 0, None, None) == L.DASH_OK  # nothing kept
    h = lib.dash_attn_active_varlen
    a = dict(Qa=FAKE, q_pos=None, cu_q=FAKE, n=40, K=FAKE, V=FAKE, mode=L.DASH_KV_ACTIVE, cu_kv=None, kvt=0,
             Oa=FAKE, Wo=None, Ua=None, score=None, ws=None, wsb=0)
    call = lambda **kw: h(None, ctypes.byref(s), *dict(a, **kw).values(), None)
    assert call(n=3 * 64 + 1) == L.DASH_E_SHAPE
    assert call(cu_q=None) == L.DASH_E_INVAL
    assert call(mode=L.DASH_KV_ALL) == L.DASH_E_INVAL  # needs q_pos and cu_kv
    assert call(mode=L.DASH_KV_ALL, q_pos=FAKE, cu_kv=FAKE, kvt=0) == L.DASH_E_SHAPE
    assert call(cu_kv=FAKE + 64) == L.DASH_E_INVAL  # active keys follow the queries
    assert call(Ua=FAKE) == L.DASH_E_INVAL
    assert call(n=0) == L.DASH_OK


def test_decode_validation(lib):
    f = lib.dash_decode
    s = _shape(B=2, S=128, Hq=28, Hkv=4)
    need = lib.dash_workspace_size(None, L.DASH_OP_DECODE, ctypes.byref(s), 1)
    assert need > 0
    args = lambda **kw: dict(dict(Qd=FAKE, n_new=1, K=FAKE, V=FAKE, n_kv=FAKE, Od=FAKE, ws=FAKE, wsb=need), **kw)
    call = lambda shape, a: f(None, ctypes.byref(shape), *a.values(), None)
    assert call(_shape(B=2, S=128, Hq=28, Hkv=4, dtype=L.DASH_F32, D=64), args()) == L.DASH_E_DTYPE
    assert call(s, args(n_new=5)) == L.DASH_E_SHAPE  # 7 * 5 rows > 32
    assert call(s, args(n_new=0)) == L.DASH_E_INVAL
    assert call(s, args(n_kv=None)) == L.DASH_E_INVAL
    assert call(s, args(wsb=need - 1)) == L.DASH_E_WORKSPACE


def test_attn_active_validation(lib):
    f = lib.dash_attn_active
    s = _shape()
    args = lambda **kw: dict(dict(Qa=FAKE, q_pos=None, n_dev=None, n_max=32, K=FAKE, V=FAKE, mode=L.DASH_KV_ACTIVE,
                                  Oa=FAKE, Wo=None, Ua=None, score=None, ws=None, wsb=0), **kw)
    call = lambda shape, a: f(None, ctypes.byref(shape), a["Qa"], a["q_pos"], a["n_dev"], a["n_max"], a["K"], a["V"],
                               a["mode"], a["Oa"], a["Wo"], a["Ua"], a["score"], a["ws"], a["wsb"], None)
    assert call(_shape(B=2), args(n_dev=FAKE)) == L.DASH_E_SHAPE  # a device row count needs B == 1
    assert "B == 1" in _last(lib)
    assert call(s, args(mode=5)) == L.DASH_E_INVAL
    assert call(s, args(n_max=65)) == L.DASH_E_INVAL
    assert call(s, args(mode=L.DASH_KV_ALL)) == L.DASH_E_INVAL
    assert "q_pos" in _last(lib)
    assert call(s, args(Ua=FAKE)) == L.DASH_E_INVAL
    assert call(s, args(Wo=FAKE, Ua=FAKE, score=FAKE)) == L.DASH_E_WORKSPACE
    assert call(s, args(Qa=None)) == L.DASH_E_INVAL
    assert call(s, args(n_max=0, Qa=None)) == L.DASH_OK


def test_attn_active_gather_validation(lib):
    """The gather variant rejects a missing q_rows and otherwise validates like
    dash_attn_active (all before any launch)."""
    f = lib.dash_attn_active_gather
    s = _shape()
    args = lambda **kw: dict(dict(Q=FAKE, q_rows=FAKE, q_pos=None, n_dev=None, n_max=32, K=FAKE, V=FAKE,
                                  mode=L.DASH_KV_ACTIVE, Oa=FAKE, Wo=None, Ua=None, score=None, ws=None, wsb=0), **kw)
    call = lambda shape, a: f(None, ctypes.byref(shape), a["Q"], a["q_rows"], a["q_pos"], a["n_dev"], a["n_max"],
                               a["K"], a["V"], a["mode"], a["Oa"], a["Wo"], a["Ua"], a["score"], a["ws"], a["wsb"],
                               None)
    assert call(s, args(q_rows=None)) == L.DASH_E_INVAL
    assert "q_rows" in _last(lib)
    assert call(_shape(B=2), args(n_dev=FAKE)) == L.DASH_E_SHAPE
    assert call(s, args(n_max=65)) == L.DASH_E_INVAL
    assert call(s, args(mode=L.DASH_KV_ALL)) == L.DASH_E_INVAL
    assert "q_pos" in _last(lib)
    assert call(s, args(Wo=FAKE, Ua=FAKE, score=FAKE)) == L.DASH_E_WORKSPACE
    assert call(s, args(Q=FAKE + 4)) == L.DASH_E_ALIGN
    assert call(s, args(Q=None)) == L.DASH_E_INVAL
    assert "Q is NULL" in _last(lib)
    assert call(s, args(n_max=0, Q=None)) == L.DASH_OK


def test_workspace_size(lib):
    s = _shape(hidden=3584, S=8192, Hq=28, Hkv=4)
    n = lib.dash_workspace_size(None, L.DASH_OP_ATTN_LAYER, ctypes.byref(s), 8192)
    assert n >= 8192 * 4
    # selection: one int32 NaN count per row (B rows), at least 256 bytes
    assert lib.dash_workspace_size(None, L.DASH_OP_SELECT, ctypes.byref(_shape(B=1)), 8192) == 256
    assert lib.dash_workspace_size(None, L.DASH_OP_SELECT, ctypes.byref(_shape(B=100)), 8192) == 512
    # one row longer than 32768 scores: plus the multi-workgroup top-k's scratch
    # (state 256 B; per 2048-score slice 16 B of extrema, 8 B of counts and a
    # 2048-bin histogram, each array in 256-byte granules): 131072 -> 64 slices
    assert lib.dash_workspace_size(None, L.DASH_OP_SELECT, ctypes.byref(_shape(B=1)), 32768) == 256
    assert lib.dash_workspace_size(None, L.DASH_OP_SELECT, ctypes.byref(_shape(B=1)), 131072) == \
        256 + 256 + 1024 + 512 + 64 * 2048 * 4
    assert lib.dash_workspace_size(None, L.DASH_OP_SELECT, ctypes.byref(_shape(B=2)), 131072) == 256
    assert lib.dash_workspace_size(None, 17, ctypes.byref(s), 8192) == 0
    assert lib.dash_workspace_size(None, L.DASH_OP_ATTN_LAYER, ctypes.byref(_shape(D=33)), 8192) == 0


def test_binding_refuses_host_and_strided_tensors():
    """The Python binding hands only dense device memory to the library: a host
    tensor or a strided view raises before anything reaches a kernel."""
    import torch
    import attention_delta_token_amd as dash
    idx = torch.zeros(4, dtype=torch.int32)
    X = torch.zeros(8, 16, dtype=torch.float32)
    Xa = torch.zeros(4, 16, dtype=torch.float32)
    with pytest.raises(ValueError, match="device"):
        dash.dash_compact(idx, X, Xa)
    with pytest.raises(ValueError, match="device"):
        dash.dash_select(torch.zeros(16), torch.zeros(8, dtype=torch.int32), k=8)


def test_binding_refuses_undersized_or_mistyped_buffers():
    """An output smaller than the shape the binding derives, or an argument of
    the wrong element type, raises before any pointer is taken (so before any
    kernel could write past its end)."""
    import torch
    import attention_delta_token_amd as dash
    idx = torch.zeros(4, dtype=torch.int32)
    X = torch.zeros(8, 16, dtype=torch.float32)
    with pytest.raises(ValueError, match="at least"):
        dash.dash_compact(idx, X, torch.zeros(3, 16, dtype=torch.float32))
    with pytest.raises(ValueError, match="dtype"):
        dash.dash_compact(idx.long(), X, torch.zeros(4, 16, dtype=torch.float32))
    with pytest.raises(ValueError, match="at least"):
        dash.dash_select(torch.zeros(16), torch.zeros(7, dtype=torch.int32), k=8)
    B, S, Hq, Hkv, D, hidden = 1, 64, 4, 2, 64, 128
    bf = dict(dtype=torch.bfloat16)
    Q, K, V = torch.zeros(B, S, Hq, D, **bf), torch.zeros(B, S, Hkv, D, **bf), torch.zeros(B, S, Hkv, D, **bf)
    Wo = torch.zeros(hidden, Hq * D, **bf)
    O, U = torch.zeros(B, S, Hq, D, **bf), torch.zeros(B, S, hidden, **bf)
    with pytest.raises(ValueError, match="U: .*at least"):
        dash.dash_attn_layer(Q, K, V, Wo, O, U[:, :S - 1].contiguous(), torch.zeros(B, S))
    with pytest.raises(ValueError, match="score: dtype"):
        dash.dash_attn_layer(Q, K, V, Wo, O, U, torch.zeros(B, S, **bf))
