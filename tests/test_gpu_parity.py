"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Bars (written into each test):
* selection, order statistic, threshold step and compaction: bit-exact when
  fed the same score vectors / rows;
* O and U: max|Δ| <= 2e-2 * max|ref| for bf16, <= 1e-4 * max|ref| for fp32;
* Δattn score: |Δ| <= 1e-2 * ref per token;
* end-to-end selection: a token may differ between the GPU and oracle sets
  only if its oracle score is within 1e-2 relative of the oracle's cut.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import oracle_par
from workload import WORKLOADS, SCORE_KINDS, layer_inputs, round_bf16, score_vector

pytestmark = pytest.mark.gpu

TOL_BF16 = 2e-2
TOL_F32 = 1e-4
TOL_SCORE = 1e-2


@pytest.fixture(scope="module")
def dash():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import attention_delta_token_amd as d
    d.load()
    return d


def say(*a):
    print(*a, flush=True)


def dev_t(a, dtype=torch.bfloat16):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda", dtype)


def host(t):
    return t.float().cpu().numpy() if t.dtype in (torch.bfloat16, torch.float16) else t.cpu().numpy()


def maxrel(got, ref):
    return float(np.max(np.abs(np.asarray(got, np.float64) - ref)) / np.max(np.abs(ref)))


def selection_within_cut(gpu_idx, ref_score, k, rel=TOL_SCORE):
    """Different tokens between the GPU set and the oracle set must lie within rel of the cut."""
    ref_idx = oracle.select_topk(ref_score, k)
    diff = np.setxor1d(gpu_idx, ref_idx)
    if k == 0 or diff.size == 0:
        return 0
    cut = np.sort(ref_score)[::-1][k - 1]
    assert np.all(np.abs(ref_score[diff] - cut) <= rel * cut), (diff, ref_score[diff], cut)
    return int(diff.size)


# ---------------------------------------------------------------------------
# selection (bit-exact on identical score vectors)
# ---------------------------------------------------------------------------

SEL_SIZES = [1, 5, 64, 1000, 4096, 4097, 8192, 16383, 32768, 32769, 65536 + 17, 131072]


@pytest.mark.parametrize("n", SEL_SIZES)
@pytest.mark.parametrize("kind", SCORE_KINDS)
def test_topk_bit_exact(dash, kind, n):
    s = score_vector(kind, n, seed=n + 1)
    sd = torch.from_numpy(s).cuda()
    for k in sorted({0, 1, n // 3, n // 2, n - 1, n} & set(range(n + 1))):
        say("topk", kind, n, k)
        idx = torch.full((max(k, 1),), -7, dtype=torch.int32, device="cuda")
        dash.dash_select(sd, idx, mode=dash.DASH_SEL_TOPK, k=k)
        torch.cuda.synchronize()
        exp = oracle.select_topk(s, k)
        np.testing.assert_array_equal(idx.cpu().numpy()[:k], exp)


@pytest.mark.parametrize("n_max,n,with_pos", [(40000, 40000, False), (65536, 65536, True), (65536, 33000, True),
                                               (131072, 100001, True), (70000, 0, True)])
def test_threshold_step_multi_workgroup(dash, n_max, n, with_pos):
    """Threshold steps over more than 32768 rows with a workspace large enough
    for the multi-workgroup kernels: survivors, counters, survivor count and
    NaN count bit-exact against the oracle's step and against the
    one-workgroup kernel (no workspace); device row count, positions outside
    the counters (dropped), NaN scores, two steps in a row."""
    rng = np.random.default_rng(n_max + n)
    S = n_max + 5000
    s = np.abs(rng.standard_normal(n_max)).astype(np.float32)
    s[rng.choice(n_max, 50, replace=False)] = np.nan
    if with_pos:
        posv = np.sort(rng.choice(S, n_max, replace=False)).astype(np.int32)
        posv[-3:] = [S + 1, S + 9, -4][: min(3, n_max)]  # outside the counters: dropped
    else:
        posv = np.arange(n_max, dtype=np.int32)
    S_c = S if with_pos else n_max
    c0 = rng.integers(0, 3, S_c).astype(np.uint8)
    tau = np.float32(0.6)
    sd = torch.from_numpy(s).cuda()
    pd = torch.from_numpy(posv).cuda() if with_pos else None
    nd = torch.tensor([n], dtype=torch.int32, device="cuda")
    tdev = torch.tensor([tau], device="cuda")
    say("threshold multi", n_max, n, with_pos)
    outs = []
    for status in (dash.select_status(1, n_max=n_max), None):
        cnt = torch.from_numpy(c0.copy()).cuda()
        for _ in range(2):
            out = torch.full((n_max,), -7, dtype=torch.int32, device="cuda")
            nout = torch.zeros(1, dtype=torch.int32, device="cuda")
            st = status if status is not None else dash.select_status(1)
            dash.dash_select(sd, out, mode=dash.DASH_SEL_THRESHOLD, tau=tdev, patience=2, counters=cnt, pos=pd,
                             n_dev=nd, n_max=n_max, n_out=nout, status=st)
        torch.cuda.synchronize()
        outs.append((out.cpu().numpy()[: int(nout.item())], cnt.cpu().numpy(), int(st[0].item())))
    # the oracle: two steps over the first n rows (positions outside the counters dropped)
    rows = posv[:n]
    keep_rows = (rows >= 0) & (rows < S_c)
    c = c0.copy()
    for _ in range(2):
        exp_pos, c_new = oracle.threshold_step(s[:n][keep_rows], rows[keep_rows], c, tau, 2)
        c = c_new
    np.testing.assert_array_equal(outs[0][0], exp_pos)
    np.testing.assert_array_equal(outs[0][1], c)
    assert outs[0][2] == int(np.isnan(s[:n]).sum())
    for a, b in zip(outs[0], outs[1]):
        np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("n", [32769, 40000, 65536 + 17, 131072, 262144 + 5])
@pytest.mark.parametrize("kind", SCORE_KINDS)
def test_topk_long_row_multi_workgroup(dash, kind, n):
    """One row longer than 32768 scores with a workspace large enough for the
    multi-workgroup top-k: bit-exact against the oracle for k from 1 to n,
    with forced ends and a position map, NaN count in the status word; the
    same outputs as the one-workgroup kernel (no workspace)."""
    s = score_vector(kind, n, seed=7 * n + 1)
    sd = torch.from_numpy(s).cuda()
    st = dash.select_status(1, n_max=n)
    for k, f, l in ((1, 0, 0), (n // 3, 0, 0), (n // 2 + 1, 0, 0), (n - 1, 0, 0), (n, 0, 0), (4096, 64, 32),
                    (n - 5, 3, 2)):
        say("topk long row", kind, n, k, f, l)
        st.fill_(-1)
        idx = torch.full((k,), -7, dtype=torch.int32, device="cuda")
        dash.dash_select(sd, idx, mode=dash.DASH_SEL_TOPK, k=k, keep_first=f, keep_last=l, status=st)
        ref = torch.full((k,), -9, dtype=torch.int32, device="cuda")
        dash.dash_select(sd, ref, mode=dash.DASH_SEL_TOPK, k=k, keep_first=f, keep_last=l)
        torch.cuda.synchronize()
        got = idx.cpu().numpy()
        np.testing.assert_array_equal(got, oracle.select_topk_forced(s, k, f, l))
        np.testing.assert_array_equal(got, ref.cpu().numpy())
        assert int(st[0].item()) == int(np.isnan(s).sum())
    # position map (the multi-shot layout): positions are pos[i]
    pos = torch.from_numpy(np.arange(n, dtype=np.int32) * 3 + 11).cuda()
    k = n // 4
    idx = torch.empty(k, dtype=torch.int32, device="cuda")
    dash.dash_select(sd, idx, mode=dash.DASH_SEL_TOPK, k=k, pos=pos, status=st)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(idx.cpu().numpy(), oracle.select_topk(s, k) * 3 + 11)


@pytest.mark.parametrize("n", [8192, 8188, 4100, 4096, 2052, 2048, 1028, 1024, 1020, 500])
@pytest.mark.parametrize("kind", SCORE_KINDS)
def test_topk_wave_rows_all_kinds(dash, kind, n):
    """The one-wave-per-row batch path on every score family, rows that fill
    their 256-score chunks (8192, 4096, 2048, 1024) and rows that do not (4100
    and 2052: the smallest rows of the bracketed path for 32 and 16 chunks per
    lane, whose sample holds partly filled chunks); k from 1 to
    n, so cuts fall inside runs of equal scores (fewvalues, equal, bf16ties)
    as well as between distinct ones.  NaN counts per row checked too."""
    rows = 256
    s = np.stack([score_vector(kind, n, seed=1000 * r + n) for r in range(rows)])
    sd = torch.from_numpy(s).cuda()
    for k in (1, n // 3, n // 2 + 1, n - 1, n):
        say("topk wave rows", kind, n, k)
        idx = torch.full((rows, k), -7, dtype=torch.int32, device="cuda")
        st = dash.select_status(rows)
        dash.dash_select(sd, idx, mode=dash.DASH_SEL_TOPK, k=k, n_max=n, rows=rows, status=st)
        torch.cuda.synchronize()
        got = idx.cpu().numpy()
        np.testing.assert_array_equal(st.cpu().numpy()[:rows], np.isnan(s).sum(axis=1))
        for r in range(0, rows, 5):
            np.testing.assert_array_equal(got[r], oracle.select_topk(s[r], k))


@pytest.mark.parametrize("n", [65536, 40004, 32772])
@pytest.mark.parametrize("kind", SCORE_KINDS)
def test_topk_strided_rows_all_kinds(dash, kind, n):
    """Batches of rows wider than 32768 scores (plain rows, n % 4 == 0) take the
    register-resident workgroup kernel with strided key ownership: every score
    family, k from 1 to n, NaN counts per row."""
    rows = 3
    s = np.stack([score_vector(kind, n, seed=7000 * r + n) for r in range(rows)])
    sd = torch.from_numpy(s).cuda()
    for k in (1, n // 3, n // 2 + 1, n - 1, n):
        say("topk strided rows", kind, n, k)
        idx = torch.full((rows, k), -7, dtype=torch.int32, device="cuda")
        st = dash.select_status(rows)
        dash.dash_select(sd, idx, mode=dash.DASH_SEL_TOPK, k=k, n_max=n, rows=rows, status=st)
        torch.cuda.synchronize()
        got = idx.cpu().numpy()
        np.testing.assert_array_equal(st.cpu().numpy()[:rows], np.isnan(s).sum(axis=1))
        for r in range(rows):
            np.testing.assert_array_equal(got[r], oracle.select_topk(s[r], k))


@pytest.mark.parametrize("n", [8192, 8188, 4096, 4092])
def test_topk_wave_rows_sample_misleads(dash, n):
    """Rows whose sampled chunks (the even 256-score chunks of a row held by
    one wave) hold only small scores while the odd chunks hold large ones: the
    sample's estimate of the cut is far off, the bracket misses and the row
    takes the digit passes over all its keys.  Mixed in a batch with random
    rows, which take the bracket; every row bit-exact against the oracle,
    including cuts inside runs of equal scores."""
    rows = 256
    g = np.random.default_rng(n)
    s = g.random((rows, n), dtype=np.float32)
    pos = np.arange(n)
    odd = ((pos // 256) % 2) == 1
    for r in range(0, rows, 2):
        s[r, odd] += 10.0
    for r in range(1, rows, 4):  # ties: few distinct values in the odd rows' upper half
        s[r, n // 2:] = np.floor(s[r, n // 2:] * 4.0)
    sd = torch.from_numpy(s).cuda()
    for k in (1, n // 3, n // 2 - 7, n - 1):
        say("topk sample misleads", n, k)
        idx = torch.full((rows, k), -7, dtype=torch.int32, device="cuda")
        dash.dash_select(sd, idx, mode=dash.DASH_SEL_TOPK, k=k, n_max=n, rows=rows)
        torch.cuda.synchronize()
        got = idx.cpu().numpy()
        for r in range(rows):
            np.testing.assert_array_equal(got[r], oracle.select_topk(s[r], k))


@pytest.mark.parametrize("rows,n,k", [(48, 3000, 1234), (80, 3000, 1234), (70, 8192, 4096), (64, 8193, 100),
                                      (66, 1, 1), (65, 40000, 39999),
                                      (256, 8192, 4096), (300, 2048, 1000), (257, 4, 2), (512, 4100, 1),
                                      (256, 12, 12), (264, 1000, 999), (256, 3001, 100), (256, 8196, 77)])
def test_topk_batched_rows(dash, rows, n, k):
    """Batches of independent rows: from 256 rows of at most 8192 scores (n % 4 == 0)
    one wave per row; otherwise one 1024-thread workgroup per row."""
    s = np.stack([score_vector("fewvalues" if r % 2 else ("bf16ties" if r % 3 else "normal"), n, seed=r)
                  for r in range(rows)])
    idx = torch.empty(rows, k, dtype=torch.int32, device="cuda")
    say("topk batched", rows, n, k)
    dash.dash_select(torch.from_numpy(s).cuda(), idx, mode=dash.DASH_SEL_TOPK, k=k, n_max=n, rows=rows)
    torch.cuda.synchronize()
    got = idx.cpu().numpy()
    for r in range(rows):
        np.testing.assert_array_equal(got[r], oracle.select_topk(s[r], k))


def test_topk_pos_map(dash):
    n, k = 5000, 1700
    s = score_vector("perm", n, seed=3)
    pos = np.sort(np.random.default_rng(0).choice(20000, n, replace=False)).astype(np.int32)
    idx = torch.empty(k, dtype=torch.int32, device="cuda")
    dash.dash_select(torch.from_numpy(s).cuda(), idx, mode=dash.DASH_SEL_TOPK, k=k, pos=torch.from_numpy(pos).cuda())
    torch.cuda.synchronize()
    np.testing.assert_array_equal(idx.cpu().numpy(), pos[oracle.select_topk(s, k)])


def _forced_cases(n):
    """(keep_first, keep_last) pairs with f + l <= n, including the pages' defaults 64 / 32."""
    pairs = [(0, 1), (1, 0), (64, 32), (5, 0), (0, 7), (n // 2, n - n // 2)]
    return sorted({(f, l) for f, l in pairs if f + l <= n})


@pytest.mark.parametrize("n", [1, 97, 4096 + 96, 8192, 32768 + 96, 65536 + 17, 131072])
@pytest.mark.parametrize("kind", ["normal", "equal", "bf16ties", "special", "decreasing"])
def test_topk_forced_bit_exact(dash, kind, n):
    """Forced retention of the first/last tokens: bit-exact against the oracle for
    k from f + l (nothing chosen by score) through the pages' K_eff to n."""
    s = score_vector(kind, n, seed=7 * n + 3)
    sd = torch.from_numpy(s).cuda()
    for f, l in _forced_cases(n):
        ks = {f + l, min(n, f + l + 1), oracle.effective_keep_count(n, 0.333, f, l), n}
        for k in sorted(ks):
            say("topk forced", kind, n, f, l, k)
            idx = torch.full((max(k, 1),), -7, dtype=torch.int32, device="cuda")
            dash.dash_select(sd, idx, mode=dash.DASH_SEL_TOPK, k=k, keep_first=f, keep_last=l)
            torch.cuda.synchronize()
            np.testing.assert_array_equal(idx.cpu().numpy()[:k], oracle.select_topk_forced(s, k, f, l))


@pytest.mark.parametrize("rows", [24, 70])
def test_topk_forced_batched_and_pos(dash, rows):
    n, f, l = 3000, 64, 32
    k = oracle.effective_keep_count(n, 0.333, f, l)
    assert k == dash.keep_count(n, 0.333, f, l)
    s = np.stack([score_vector("fewvalues" if r % 2 else "normal", n, seed=100 + r) for r in range(rows)])
    idx = torch.empty(rows, k, dtype=torch.int32, device="cuda")
    say("topk forced batched", rows, n, k)
    dash.dash_select(torch.from_numpy(s).cuda(), idx, mode=dash.DASH_SEL_TOPK, k=k, n_max=n, rows=rows,
                     keep_first=f, keep_last=l)
    torch.cuda.synchronize()
    got = idx.cpu().numpy()
    for r in range(rows):
        np.testing.assert_array_equal(got[r], oracle.select_topk_forced(s[r], k, f, l))
    pos = np.sort(np.random.default_rng(1).choice(20000, n, replace=False)).astype(np.int32)
    idx1 = torch.empty(k, dtype=torch.int32, device="cuda")
    dash.dash_select(torch.from_numpy(s[0]).cuda(), idx1, mode=dash.DASH_SEL_TOPK, k=k, keep_first=f, keep_last=l,
                     pos=torch.from_numpy(pos).cuda())
    torch.cuda.synchronize()
    np.testing.assert_array_equal(idx1.cpu().numpy(), pos[oracle.select_topk_forced(s[0], k, f, l)])


@pytest.mark.parametrize("n", [1, 50, 4097, 65536])
@pytest.mark.parametrize("kind", SCORE_KINDS)
def test_order_statistic_bit_exact(dash, kind, n):
    s = score_vector(kind, n, seed=2 * n + 5)
    sd = torch.from_numpy(s).cuda()
    tau = torch.empty(4, dtype=torch.float32, device="cuda")
    for r in sorted({1, oracle.percentile_rank(n, 30), n}):
        say("order stat", kind, n, r)
        dash.dash_select(sd, mode=dash.DASH_SEL_ORDER_STAT, rank=r, tau_out=tau)
        torch.cuda.synchronize()
        got = float(tau[0].item())
        exp = np.float32(oracle.order_statistic(s, r))
        if math.isnan(exp):
            assert math.isnan(got)
        else:
            assert np.float32(got).tobytes() == exp.tobytes(), (got, exp)


def test_order_statistic_device_count(dash):
    n_max, n = 9000, 6123
    s = score_vector("normal", n_max, seed=9)
    nd = torch.tensor([n, 0, 0, 0], dtype=torch.int32, device="cuda")
    tau = torch.empty(4, dtype=torch.float32, device="cuda")
    for r in (1, 1837, n, n + 1):
        dash.dash_select(torch.from_numpy(s).cuda(), mode=dash.DASH_SEL_ORDER_STAT, rank=r, n_dev=nd, n_max=n_max,
                         tau_out=tau)
        torch.cuda.synchronize()
        got = float(tau[0].item())
        if r > n:
            assert math.isnan(got)  # rank beyond the device count
        else:
            assert np.float32(got) == np.float32(oracle.order_statistic(s[:n], r))


@pytest.mark.parametrize("n_max,n,S", [(1, 1, 1), (700, 700, 700), (5000, 3210, 9000), (70000, 65536, 70000)])
@pytest.mark.parametrize("with_pos", [False, True])
def test_threshold_step_bit_exact(dash, n_max, n, S, with_pos):
    rng = np.random.default_rng(n + S)
    if not with_pos:
        S = n_max
    pos = np.sort(rng.choice(S, n_max, replace=False)).astype(np.int32) if with_pos else np.arange(n_max, dtype=np.int32)
    s = score_vector("special" if n % 2 else "normal", n_max, seed=n)
    counters = rng.integers(0, 2, S).astype(np.uint8)
    tau = np.float32(0.7)
    say("threshold", n_max, n, S, with_pos)
    cd = torch.from_numpy(counters.copy()).cuda()
    out = torch.full((n_max,), -5, dtype=torch.int32, device="cuda")
    nout = torch.full((4,), -1, dtype=torch.int32, device="cuda")
    nd = torch.tensor([n, 0, 0, 0], dtype=torch.int32, device="cuda")
    taud = torch.tensor([tau, 0, 0, 0], dtype=torch.float32, device="cuda")
    dash.dash_select(torch.from_numpy(s).cuda(), out, mode=dash.DASH_SEL_THRESHOLD, tau=taud, patience=2,
                     counters=cd, pos=torch.from_numpy(pos).cuda() if with_pos else None, n_dev=nd, n_max=n_max,
                     n_out=nout)
    torch.cuda.synchronize()
    exp_pos, exp_c = oracle.threshold_step(s[:n], pos[:n], counters, float(tau), 2)
    m = int(nout[0].item())
    assert m == exp_pos.shape[0]
    np.testing.assert_array_equal(out.cpu().numpy()[:m], exp_pos)
    np.testing.assert_array_equal(cd.cpu().numpy(), exp_c)
    assert np.all(out.cpu().numpy()[m:] == -5)


def test_threshold_chain_of_layers(dash):
    """Several consecutive layers with device-resident counts, as the stack runs them."""
    S, L_ = 3000, 6
    rng = np.random.default_rng(11)
    scores = rng.random((L_, S)).astype(np.float32)
    tau = np.float32(0.45)
    taud = torch.tensor([tau, 0, 0, 0], device="cuda")
    cd = torch.zeros(S, dtype=torch.uint8, device="cuda")
    bufs = [torch.arange(S, dtype=torch.int32, device="cuda"), torch.empty(S, dtype=torch.int32, device="cuda")]
    ns = [torch.tensor([S, 0, 0, 0], dtype=torch.int32, device="cuda"), torch.zeros(4, dtype=torch.int32, device="cuda")]
    pos_h, c_h = np.arange(S, dtype=np.int32), np.zeros(S, dtype=np.uint8)
    cur = 0
    for l in range(L_):
        row = scores[l][pos_h]  # the scores of the active rows, in active order
        srow = torch.zeros(S, dtype=torch.float32, device="cuda")
        srow[: row.shape[0]] = torch.from_numpy(row).cuda()
        dash.dash_select(srow, bufs[cur ^ 1], mode=dash.DASH_SEL_THRESHOLD, tau=taud, patience=2, counters=cd,
                         pos=bufs[cur], n_dev=ns[cur], n_max=S, n_out=ns[cur ^ 1])
        pos_h, c_h = oracle.threshold_step(row, pos_h, c_h, float(tau), 2)
        cur ^= 1
        torch.cuda.synchronize()
        m = int(ns[cur][0].item())
        np.testing.assert_array_equal(bufs[cur].cpu().numpy()[:m], pos_h)
        np.testing.assert_array_equal(cd.cpu().numpy(), c_h)


def test_threshold_positions_outside_counters_are_dropped(dash):
    """A row whose position lies outside the counters array is not emitted and
    touches no counter; the other rows follow the threshold step unchanged."""
    n, n_counters = 3000, 2500
    rng = np.random.default_rng(21)
    pos = np.sort(rng.choice(3400, n, replace=False)).astype(np.int32)  # some positions >= n_counters
    s = score_vector("normal", n, seed=21)
    counters = rng.integers(0, 2, n_counters).astype(np.uint8)
    tau = np.float32(0.6)
    cd = torch.from_numpy(counters.copy()).cuda()
    out = torch.full((n,), -5, dtype=torch.int32, device="cuda")
    nout = torch.zeros(4, dtype=torch.int32, device="cuda")
    dash.dash_select(torch.from_numpy(s).cuda(), out, mode=dash.DASH_SEL_THRESHOLD,
                     tau=torch.tensor([tau], device="cuda"), patience=2, counters=cd,
                     pos=torch.from_numpy(pos).cuda(), n_max=n, n_out=nout)
    torch.cuda.synchronize()
    inside = pos < n_counters
    assert not np.all(inside)
    exp_pos, exp_c = oracle.threshold_step(s[inside], pos[inside], counters, float(tau), 2)
    m = int(nout[0].item())
    assert m == exp_pos.shape[0]
    np.testing.assert_array_equal(out.cpu().numpy()[:m], exp_pos)
    np.testing.assert_array_equal(cd.cpu().numpy(), exp_c)


@pytest.mark.parametrize("n_max", [5000, 70000])
def test_topk_device_count(dash, n_max):
    """Top-k over the first n = *n_dev scores of a row of capacity n_max: min(k, n)
    kept (forced ends shrink with it), the kept count written to n_out, the
    outputs past it untouched; bit-exact against the oracle on the first n."""
    s = score_vector("bf16ties", n_max, seed=n_max)
    sd = torch.from_numpy(s).cuda()
    for n in (0, 1, 777, n_max - 1234, n_max, n_max + 9):
        for k, f, l in ((100, 0, 0), (2000, 64, 32), (n_max - 1, 0, 0), (0, 0, 0), (40, 30, 10)):
            nc = min(max(n, 0), n_max)
            kk = min(k, nc)
            ff = min(f, kk)
            ll = min(l, kk - ff)
            say("topk device count", n_max, n, k, f, l)
            idx = torch.full((max(k, 1),), -7, dtype=torch.int32, device="cuda")
            nd = torch.tensor([n], dtype=torch.int32, device="cuda")
            nout = torch.full((1,), -1, dtype=torch.int32, device="cuda")
            st = dash.select_status(1)
            dash.dash_select(sd, idx, mode=dash.DASH_SEL_TOPK, k=k, n_dev=nd, n_max=n_max, n_out=nout,
                             keep_first=f, keep_last=l, status=st)
            torch.cuda.synchronize()
            assert int(nout[0].item()) == kk
            got = idx.cpu().numpy()
            np.testing.assert_array_equal(got[:kk], oracle.select_topk_forced(s[:nc], kk, ff, ll))
            assert np.all(got[kk:k] == -7)
            assert int(st[0].item()) == 0


def test_select_nan_status(dash):
    """The NaN count of every selection mode (one int32 per row in the
    workspace) equals the number of NaN scores the call ranks or updates."""
    def nans(a):
        return int(np.isnan(a).sum())
    # single rows: register-resident (<= 32768) and long rows, plain and forced
    for n in (1, 4097, 32768, 65536 + 17):
        s = score_vector("special", n, seed=n + 3)
        sd = torch.from_numpy(s).cuda()
        for k, f, l in ((n // 2, 0, 0), (n, 0, 0), (min(n, 200), min(n, 64), 0), (0, 0, 0)):
            st = torch.full((64,), -1, dtype=torch.int32, device="cuda")
            idx = torch.empty(max(k, 1), dtype=torch.int32, device="cuda")
            dash.dash_select(sd, idx, mode=dash.DASH_SEL_TOPK, k=k, keep_first=f, keep_last=l, status=st)
            torch.cuda.synchronize()
            assert int(st[0].item()) == nans(s), (n, k, f)
            if k:
                np.testing.assert_array_equal(idx.cpu().numpy()[:k], oracle.select_topk_forced(s, k, f, l))
        tau = torch.empty(1, dtype=torch.float32, device="cuda")
        st = torch.full((64,), -1, dtype=torch.int32, device="cuda")
        dash.dash_select(sd, mode=dash.DASH_SEL_ORDER_STAT, rank=max(1, n // 3), tau_out=tau, status=st)
        torch.cuda.synchronize()
        assert int(st[0].item()) == nans(s)
        st = torch.full((64,), -1, dtype=torch.int32, device="cuda")
        out = torch.empty(n, dtype=torch.int32, device="cuda")
        nout = torch.zeros(1, dtype=torch.int32, device="cuda")
        cnt = torch.zeros(n, dtype=torch.uint8, device="cuda")
        dash.dash_select(sd, out, mode=dash.DASH_SEL_THRESHOLD, tau=torch.tensor([0.3], device="cuda"), patience=2,
                         counters=cnt, n_max=n, n_out=nout, status=st)
        torch.cuda.synchronize()
        assert int(st[0].item()) == nans(s)
        exp_pos, exp_c = oracle.threshold_step(s, np.arange(n), np.zeros(n, np.uint8), 0.3, 2)
        np.testing.assert_array_equal(out.cpu().numpy()[:int(nout[0].item())], exp_pos)
    # batches: one wave per row (>= 256 rows of <= 8192) and one workgroup per row
    for rows, n in ((300, 2048), (40, 3000)):
        s = np.stack([score_vector("special" if r % 3 else "normal", n, seed=r) for r in range(rows)])
        st = dash.select_status(rows)
        idx = torch.empty(rows, n // 2, dtype=torch.int32, device="cuda")
        dash.dash_select(torch.from_numpy(s).cuda(), idx, mode=dash.DASH_SEL_TOPK, k=n // 2, n_max=n, rows=rows,
                         status=st)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(st.cpu().numpy()[:rows], np.isnan(s).sum(axis=1))
        got = idx.cpu().numpy()
        for r in range(0, rows, 7):
            np.testing.assert_array_equal(got[r], oracle.select_topk(s[r], n // 2))


# ---------------------------------------------------------------------------
# compaction (bit-exact)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("row_bytes", [16, 48, 1024, 1040, 2048, 2064, 7168])
@pytest.mark.parametrize("device_n", [False, True])
def test_compact_bit_exact(dash, row_bytes, device_n):
    S, n_max = 3001, 1500
    rng = np.random.default_rng(row_bytes)
    X = rng.integers(0, 256, (S, row_bytes), dtype=np.uint8)
    idx = np.sort(rng.choice(S, n_max, replace=False)).astype(np.int32)
    n = 1234 if device_n else n_max
    Xa = torch.full((n_max, row_bytes), 0xAB, dtype=torch.uint8, device="cuda")
    say("compact", row_bytes, device_n)
    nd = torch.tensor([n, 0, 0, 0], dtype=torch.int32, device="cuda") if device_n else None
    dash.dash_compact(torch.from_numpy(idx).cuda(), torch.from_numpy(X).cuda(), Xa, n_dev=nd, n_max=n_max)
    torch.cuda.synchronize()
    got = Xa.cpu().numpy()
    np.testing.assert_array_equal(got[:n], oracle.compact(X, idx[:n]))
    assert np.all(got[n:] == 0xAB)


@pytest.mark.parametrize("widths", [(7168, 1024, 1024), (16,), (48, 16, 7168, 32), (1024, 48), (2048,),
                                    (2048, 1040, 16), (1024, 1024, 512, 16), (2048, 2048, 2048, 1024)])
@pytest.mark.parametrize("device_n", [False, True])
def test_compact_many_bit_exact(dash, widths, device_n):
    """Several tensors of different row widths gathered at one index list in one
    launch; idx holds out-of-range entries (those rows are not copied)."""
    S, n_max = 2049, 1100
    rng = np.random.default_rng(sum(widths))
    Xs = [rng.integers(0, 256, (S, w), dtype=np.uint8) for w in widths]
    idx = np.sort(rng.choice(S, n_max, replace=False)).astype(np.int32)
    idx[[5, 700]] = [-1, S + 3]  # skipped rows
    n = 987 if device_n else n_max
    Xas = [torch.full((n_max, w), 0xCD, dtype=torch.uint8, device="cuda") for w in widths]
    say("compact many", widths, device_n)
    nd = torch.tensor([n, 0, 0, 0], dtype=torch.int32, device="cuda") if device_n else None
    dash.dash_compact_many(torch.from_numpy(idx).cuda(), [(torch.from_numpy(X).cuda(), Xa) for X, Xa in zip(Xs, Xas)],
                           n_dev=nd, n_max=n_max)
    torch.cuda.synchronize()
    ok = (idx[:n] >= 0) & (idx[:n] < S)
    for X, Xa in zip(Xs, Xas):
        got = Xa.cpu().numpy()
        np.testing.assert_array_equal(got[:n][ok], oracle.compact(X, idx[:n][ok]))
        assert np.all(got[:n][~ok] == 0xCD) and np.all(got[n:] == 0xCD)


@pytest.mark.parametrize("dtype,hidden", [("bf16", 3584), ("bf16", 4096), ("bf16", 8), ("bf16", 264),
                                          ("f32", 256), ("f32", 4)])
@pytest.mark.parametrize("n,device_n", [(1, False), (1000, False), (8193, True)])
def test_score_standalone(dash, dtype, hidden, n, device_n):
    """score[t] = ||U_t||_2 from a given U, against the oracle's definition; fp32
    sums of `hidden` positive terms: relative error below hidden * 2^-24."""
    rng = np.random.default_rng(hidden + n)
    U = (rng.standard_normal((n, hidden)) * rng.lognormal(0, 1, (n, 1))).astype(np.float32)
    if dtype == "bf16":
        U = round_bf16(U)
    Ud = torch.from_numpy(U).to("cuda", torch.bfloat16 if dtype == "bf16" else torch.float32)
    score = torch.full((n,), -1.0, dtype=torch.float32, device="cuda")
    m = n - 7 if device_n else n
    nd = torch.tensor([m, 0, 0, 0], dtype=torch.int32, device="cuda") if device_n else None
    say("score standalone", dtype, hidden, n, device_n)
    dash.dash_score(Ud, score, n_dev=nd, n_max=n)
    torch.cuda.synchronize()
    got = score.cpu().numpy()
    ref = oracle.delta_attn(U[:m])
    assert np.all(np.abs(got[:m] - ref) <= max(hidden, 16) * 2.0 ** -24 * ref)
    assert np.all(got[m:] == -1.0)


# ---------------------------------------------------------------------------
# attention + projection + score
# ---------------------------------------------------------------------------

def _layer(S, Hq, Hkv, D, hidden, seed, dtype="bf16"):
    w = WORKLOADS[1].scaled(S=S, Hq=Hq, Hkv=Hkv, D=D, hidden=hidden, dtype=dtype)
    return layer_inputs(w, seed, 0)


def _run_layer(dash, x, dtype=torch.bfloat16, with_score=True):
    S, Hq, D = x["Q"].shape
    hidden = x["Wo"].shape[1]
    Q, K, V = (dev_t(x[n], dtype) for n in ("Q", "K", "V"))
    Wo = dev_t(x["Wo"].T, dtype)
    O = torch.empty(S, Hq * D, device="cuda", dtype=dtype)
    U = torch.empty(S, hidden, device="cuda", dtype=dtype)
    score = torch.empty(S, device="cuda", dtype=torch.float32) if with_score else None
    dc = dash.DASH_BF16 if dtype == torch.bfloat16 else dash.DASH_F32
    ws = dash.workspace(dash.DASH_OP_ATTN_LAYER, dash.make_shape(1, S, Hq, x["K"].shape[1], D, hidden, dc), S)
    dash.dash_attn_layer(Q, K, V, Wo, O, U, score, ws)
    torch.cuda.synchronize()
    return host(O), host(U), (host(score) if with_score else None)


@pytest.mark.parametrize("S,Hq,Hkv,D,hidden", [
    (1, 2, 1, 128, 256), (77, 4, 2, 64, 128), (300, 8, 2, 128, 384), (640, 28, 4, 128, 3584),
    (1000, 32, 8, 128, 4096), (129, 7, 7, 64, 200),
    # 4096 rows x 4096 columns: the W_o GEMM launcher takes its 256-wide tiles
    # (the 224-wide grid would spill into a second wave of workgroups); the
    # shapes above take the 224-wide ones
    (4096, 32, 8, 128, 4096),
    # contraction Hq*D of one, two and three 64-wide steps (the GEMM's peeled
    # last steps with no loop iteration before them), both tile widths
    (50, 1, 1, 64, 136), (260, 2, 1, 64, 264), (300, 3, 1, 64, 520),
    (4096, 1, 1, 64, 4096), (4096, 3, 1, 64, 4096),
    # 256-wide tiles with a partial last row tile (4000 = 15 * 256 + 160)
    (4000, 4, 1, 64, 4096),
])
def test_attn_layer_bf16(dash, S, Hq, Hkv, D, hidden):
    x = _layer(S, Hq, Hkv, D, hidden, seed=S)
    say("attn_layer bf16", S, Hq, Hkv, D, hidden)
    O, U, score = _run_layer(dash, x)
    if S >= 2048:
        O_ref, U_ref, s_ref = oracle_par.layer_rows(x, np.arange(S))
    else:
        O_ref, U_ref, s_ref = oracle.attention_layer(x["Q"], x["K"], x["V"], x["Wo"])
    assert maxrel(O, O_ref) <= TOL_BF16
    assert maxrel(U, U_ref) <= TOL_BF16
    assert np.all(np.abs(score - s_ref) <= TOL_SCORE * s_ref)
    # the projection alone, from the GPU's own O (isolates the GEMM)
    U_from_O = oracle.output_projection(O, x["Wo"])
    assert maxrel(U, U_from_O) <= 1e-2


@pytest.mark.parametrize("S,Hq,Hkv,D,hidden", [(512, 4, 4, 64, 256), (100, 4, 2, 32, 64), (70, 2, 1, 128, 96)])
def test_attn_layer_fp32(dash, S, Hq, Hkv, D, hidden):
    x = _layer(S, Hq, Hkv, D, hidden, seed=S, dtype="f32")
    say("attn_layer fp32", S, Hq, Hkv, D, hidden)
    O, U, score = _run_layer(dash, x, torch.float32)
    O_ref, U_ref, s_ref = oracle.attention_layer(x["Q"], x["K"], x["V"], x["Wo"])
    assert maxrel(O, O_ref) <= TOL_F32
    assert maxrel(U, U_ref) <= TOL_F32
    assert np.all(np.abs(score - s_ref) <= TOL_SCORE * s_ref)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("mode", ["active", "all"])
@pytest.mark.parametrize("device_n", [False, True])
def test_attn_active(dash, dtype, mode, device_n):
    S, Hq, Hkv, D, hidden = 900, 8, 2, (128 if dtype == "bf16" else 64), 256
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    x = _layer(S, Hq, Hkv, D, hidden, seed=5, dtype=dtype)
    rng = np.random.default_rng(1)
    n_max = 377
    idx = np.sort(rng.choice(S, n_max, replace=False)).astype(np.int32)
    n = 301 if device_n else n_max
    say("attn_active", dtype, mode, device_n)
    Qa = dev_t(x["Q"][idx], tdt)
    K = dev_t(x["K"][idx] if mode == "active" else x["K"], tdt)
    V = dev_t(x["V"][idx] if mode == "active" else x["V"], tdt)
    Wo = dev_t(x["Wo"].T, tdt)
    Oa = torch.zeros(n_max, Hq * D, device="cuda", dtype=tdt)
    Ua = torch.zeros(n_max, hidden, device="cuda", dtype=tdt)
    sc = torch.zeros(n_max, device="cuda", dtype=torch.float32)
    dc = dash.DASH_BF16 if dtype == "bf16" else dash.DASH_F32
    ws = dash.workspace(dash.DASH_OP_ATTN_ACTIVE, dash.make_shape(1, S, Hq, Hkv, D, hidden, dc), n_max)
    nd = torch.tensor([n, 0, 0, 0], dtype=torch.int32, device="cuda") if device_n else None
    km = dash.DASH_KV_ACTIVE if mode == "active" else dash.DASH_KV_ALL
    dash.dash_attn_active(Qa, K, V, km, Oa, q_pos=torch.from_numpy(idx).cuda(), n_dev=nd, n_max=n_max, Wo=Wo, Ua=Ua,
                          score=sc, ws=ws, S=S if mode == "all" else None)
    torch.cuda.synchronize()
    if mode == "active" and device_n:
        # keys are the first n compacted rows
        ref_O = oracle.attn_active(x["Q"], x["K"], x["V"], idx[:n], "active")
    else:
        ref_O = oracle.attn_active(x["Q"], x["K"], x["V"], idx[:n], mode)
    ref_U = oracle.output_projection(ref_O, x["Wo"])
    ref_s = oracle.delta_attn(ref_U)
    assert maxrel(host(Oa)[:n], ref_O) <= tol
    assert maxrel(host(Ua)[:n], ref_U) <= tol
    assert np.all(np.abs(host(sc)[:n] - ref_s) <= TOL_SCORE * ref_s)
    assert np.all(host(Oa)[n:] == 0) and np.all(host(Ua)[n:] == 0)


@pytest.mark.parametrize("B,device_n,heads", [(1, False, (8, 2)), (1, True, (8, 2)), (3, False, (8, 2)),
                                               (1, False, (6, 6))])
@pytest.mark.parametrize("dtype", ["bf16", "bf16-d64", "f32"])
@pytest.mark.parametrize("mode", ["active", "all"])
def test_attn_active_gather_matches_compacted(dash, dtype, mode, B, device_n, heads):
    """Queries read through q_rows inside the kernel give exactly what
    compacting Q first and calling dash_attn_active gives (same kernels, same
    inputs): O, U and score bit for bit; rows past the device count untouched.
    In kv-active mode q_rows also carries two out-of-range entries, which read
    the clamped rows."""
    (Hq, Hkv), D, hidden = heads, (128 if dtype == "bf16" else 64), 256
    S = 700
    dtype = "bf16" if dtype == "bf16-d64" else dtype
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    xs = [_layer(S, Hq, Hkv, D, hidden, seed=21 + b, dtype=dtype) for b in range(B)]
    k = 333
    idx = np.stack([np.sort(np.random.default_rng(40 + b).choice(S, k, replace=False)) for b in range(B)])
    idx = idx.astype(np.int32)
    rows = idx.copy()
    if mode == "active":
        rows[0, 5], rows[-1, -1] = -3, S + 7  # clamped to 0 and S - 1
    n = 250 if device_n else k
    say("attn_active_gather", dtype, D, mode, "B", B, "device_n", device_n, "heads", heads)
    Qfull = dev_t(np.stack([x["Q"] for x in xs]), tdt)
    Qa = dev_t(np.stack([x["Q"][np.clip(rows[b], 0, S - 1)] for b, x in enumerate(xs)]), tdt)
    if mode == "active":
        K = dev_t(np.stack([x["K"][idx[b]] for b, x in enumerate(xs)]), tdt)
        V = dev_t(np.stack([x["V"][idx[b]] for b, x in enumerate(xs)]), tdt)
    else:
        K = dev_t(np.stack([x["K"] for x in xs]), tdt)
        V = dev_t(np.stack([x["V"] for x in xs]), tdt)
    Wo = dev_t(xs[0]["Wo"].T, tdt)
    if B == 1:
        Qfull, Qa, K, V = Qfull[0], Qa[0], K[0], V[0]
    lead = (B,) if B > 1 else ()
    dc = dash.DASH_BF16 if dtype == "bf16" else dash.DASH_F32
    ws = dash.workspace(dash.DASH_OP_ATTN_ACTIVE, dash.make_shape(B, S, Hq, Hkv, D, hidden, dc), k)
    km = dash.DASH_KV_ACTIVE if mode == "active" else dash.DASH_KV_ALL
    q_pos = torch.from_numpy(idx if B > 1 else idx[0]).cuda()
    q_rows = torch.from_numpy(rows if B > 1 else rows[0]).cuda()
    nd = torch.tensor([n, 0, 0, 0], dtype=torch.int32, device="cuda") if device_n else None
    outs = []
    for gather in (False, True):
        Oa = torch.zeros(*lead, k, Hq * D, device="cuda", dtype=tdt)
        Ua = torch.zeros(*lead, k, hidden, device="cuda", dtype=tdt)
        sc = torch.zeros(*lead, k, device="cuda", dtype=torch.float32)
        qp = q_pos if mode == "all" else None
        if gather:
            dash.dash_attn_active_gather(Qfull, q_rows, K, V, km, Oa, q_pos=qp, n_dev=nd, n_max=k, Wo=Wo, Ua=Ua,
                                         score=sc, ws=ws)
        else:
            dash.dash_attn_active(Qa, K, V, km, Oa, q_pos=qp, n_dev=nd, n_max=k, Wo=Wo, Ua=Ua, score=sc, ws=ws,
                                  S=S if mode == "all" else None)
        torch.cuda.synchronize()
        outs.append((Oa, Ua, sc))
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(a, b)
    Oa, Ua, _ = outs[1]
    flat_O = Oa.reshape(-1, k, Hq * D)
    assert torch.count_nonzero(flat_O[:, :n]) > 0
    assert torch.count_nonzero(flat_O[:, n:]) == 0 and torch.count_nonzero(Ua.reshape(-1, k, hidden)[:, n:]) == 0


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("mode", ["active", "all"])
def test_attn_active_batched(dash, dtype, mode):
    """B = 3 samples in one call, each with its own kept positions; every sample
    against the oracle (the samples' layers differ)."""
    B, S, Hq, Hkv, D, hidden = 3, 640, 8, 2, (128 if dtype == "bf16" else 64), 256
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    xs = [_layer(S, Hq, Hkv, D, hidden, seed=11 + b, dtype=dtype) for b in range(B)]
    Wo_h = xs[0]["Wo"]  # one weight for the batch
    k = 250
    idx = np.stack([np.sort(np.random.default_rng(b).choice(S, k, replace=False)) for b in range(B)]).astype(np.int32)
    say("attn_active batched", dtype, mode)
    Qa = dev_t(np.stack([x["Q"][idx[b]] for b, x in enumerate(xs)]), tdt)
    if mode == "active":
        K = dev_t(np.stack([x["K"][idx[b]] for b, x in enumerate(xs)]), tdt)
        V = dev_t(np.stack([x["V"][idx[b]] for b, x in enumerate(xs)]), tdt)
    else:
        K = dev_t(np.stack([x["K"] for x in xs]), tdt)
        V = dev_t(np.stack([x["V"] for x in xs]), tdt)
    Wo = dev_t(Wo_h.T, tdt)
    Oa = torch.zeros(B, k, Hq * D, device="cuda", dtype=tdt)
    Ua = torch.zeros(B, k, hidden, device="cuda", dtype=tdt)
    sc = torch.zeros(B, k, device="cuda", dtype=torch.float32)
    dc = dash.DASH_BF16 if dtype == "bf16" else dash.DASH_F32
    ws = dash.workspace(dash.DASH_OP_ATTN_ACTIVE, dash.make_shape(B, S, Hq, Hkv, D, hidden, dc), k)
    km = dash.DASH_KV_ACTIVE if mode == "active" else dash.DASH_KV_ALL
    dash.dash_attn_active(Qa, K, V, km, Oa, q_pos=torch.from_numpy(idx).cuda(), n_max=k, Wo=Wo, Ua=Ua, score=sc,
                          ws=ws, S=S if mode == "all" else None)
    torch.cuda.synchronize()
    for b, x in enumerate(xs):
        ref_O = oracle.attn_active(x["Q"], x["K"], x["V"], idx[b], mode)
        ref_U = oracle.output_projection(ref_O, Wo_h)
        ref_s = oracle.delta_attn(ref_U)
        assert maxrel(host(Oa)[b], ref_O) <= tol
        assert maxrel(host(Ua)[b], ref_U) <= tol
        assert np.all(np.abs(host(sc)[b] - ref_s) <= TOL_SCORE * ref_s)


@pytest.mark.parametrize("widths", [(7168, 1024, 1024), (48,), (16, 32), (2048, 2048), (1024, 1024, 16)])
def test_compact_batch_bit_exact(dash, widths):
    """Per-sample gathers of B = 4 samples (local positions, with out-of-range entries skipped)."""
    B, S, k = 4, 1000, 300
    rng = np.random.default_rng(len(widths))
    Xs = [rng.integers(0, 256, (B, S, w), dtype=np.uint8) for w in widths]
    idx = np.stack([np.sort(rng.choice(S, k, replace=False)) for _ in range(B)]).astype(np.int32)
    idx[1, 7] = -3
    idx[2, 100] = S
    Xas = [torch.full((B, k, w), 0xEE, dtype=torch.uint8, device="cuda") for w in widths]
    say("compact batch", widths)
    dash.dash_compact_batch(torch.from_numpy(idx).cuda(), [(torch.from_numpy(X).cuda(), Xa) for X, Xa in zip(Xs, Xas)])
    torch.cuda.synchronize()
    for X, Xa in zip(Xs, Xas):
        got = Xa.cpu().numpy()
        for b in range(B):
            ok = (idx[b] >= 0) & (idx[b] < S)
            np.testing.assert_array_equal(got[b][ok], oracle.compact(X[b], idx[b][ok]))
            assert np.all(got[b][~ok] == 0xEE)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_one_shot_step_batched(dash, dtype):
    """B = 3 samples through the one-shot stack: halting layer at full length, top-k
    per sample, one gather, post-halt layer; every sample against the oracle (the
    selection bit-exact on the GPU's own scores, the post-halt layer teacher-forced)."""
    from attention_delta_token_amd.stack import LayerTensors, OneShotStack
    B = 3
    w = WORKLOADS[0] if dtype == "f32" else WORKLOADS[1].scaled(S=768, hidden=512)
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    tol = TOL_F32 if dtype == "f32" else TOL_BF16
    hostl = [[layer_inputs(w, 20 + b, l) for b in range(B)] for l in range(2)]
    Wo = [hostl[l][0]["Wo"] for l in range(2)]  # one weight per layer, shared by the batch
    layers = [LayerTensors(*(dev_t(np.stack([h[n] for h in hostl[l]]), tdt) for n in ("Q", "K", "V")),
                           dev_t(Wo[l].T, tdt)) for l in range(2)]
    k = oracle.topk_count(w.S, w.keep)
    say("one-shot batched", dtype, w.S, k)
    st = OneShotStack(layers, halt_layer=0, keep=w.keep)
    assert st.k == k
    st.run()
    torch.cuda.synchronize()
    for b in range(B):
        x0, x1 = hostl[0][b], hostl[1][b]
        _, U_ref, s_ref = oracle.attention_layer(x0["Q"], x0["K"], x0["V"], Wo[0])
        assert maxrel(host(st.U)[b], U_ref) <= tol
        score = host(st.score)[b]
        assert np.all(np.abs(score - s_ref) <= TOL_SCORE * s_ref)
        idx = st.idx.cpu().numpy()[b]
        np.testing.assert_array_equal(idx, oracle.select_topk(score, k))
        Oa = oracle.attn_active(x1["Q"], x1["K"], x1["V"], idx, "active")
        assert maxrel(host(st.Ua)[b], oracle.output_projection(Oa, Wo[1])) <= tol
    assert np.all(st.status.cpu().numpy()[:B] == 0)  # no NaN score at the decision


@pytest.mark.parametrize("mode", ["active", "all"])
def test_gather_once_step_matches_step(dash, mode):
    """The gather-once step (one gather of a hidden-state stand-in at the halting
    layer, post-halt layers on inputs compacted beforehand) gives the post-halt
    outputs of the regular step bit for bit, and its gather is exact."""
    from attention_delta_token_amd.stack import LayerTensors, OneShotStack
    w = WORKLOADS[1].scaled(S=640, hidden=384, layers=3)
    hostl = [layer_inputs(w, 40, l) for l in range(3)]
    layers = [LayerTensors(*(dev_t(h[n]) for n in ("Q", "K", "V")), dev_t(h["Wo"].T)) for h in hostl]
    kv = dash.DASH_KV_ACTIVE if mode == "active" else dash.DASH_KV_ALL
    say("gather once", mode, w.S, w.keep)
    st = OneShotStack(layers, halt_layer=0, keep=w.keep, kv_mode=kv)
    st.run()
    torch.cuda.synchronize()
    Ua_ref, idx_ref = st.Ua.clone(), st.idx.clone()
    st.prepare_gather_once()
    st.H.copy_(torch.randn(st.S, st.hidden, generator=torch.Generator().manual_seed(1)).to("cuda", torch.bfloat16))
    st.Ua.zero_()
    st.run_gather_once()
    torch.cuda.synchronize()
    assert torch.equal(st.idx, idx_ref)
    assert torch.equal(st.Ua, Ua_ref)
    assert torch.equal(st.Ha, st.H[st.idx.long()])


def test_kv_all_at_halt_layer_equals_dense_rows(dash):
    """On the GPU: post-halt attention with all K/V at the halting layer equals the dense rows."""
    S, Hq, Hkv, D, hidden = 700, 8, 2, 128, 256
    x = _layer(S, Hq, Hkv, D, hidden, seed=8)
    O, _, _ = _run_layer(dash, x, with_score=False)
    idx = np.sort(np.random.default_rng(3).choice(S, 250, replace=False)).astype(np.int32)
    Oa = torch.empty(250, Hq * D, device="cuda", dtype=torch.bfloat16)
    dash.dash_attn_active(dev_t(x["Q"][idx]), dev_t(x["K"]), dev_t(x["V"]), dash.DASH_KV_ALL, Oa,
                          q_pos=torch.from_numpy(idx).cuda(), S=S)
    torch.cuda.synchronize()
    assert np.array_equal(host(Oa), O[idx])  # same kernel, same tiles: identical bits


# ---------------------------------------------------------------------------
# whole one-shot steps
# ---------------------------------------------------------------------------

def _stack_inputs(w, seed, dtype):
    from attention_delta_token_amd.stack import LayerTensors
    hostl = [layer_inputs(w, seed, l) for l in range(w.layers)]
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    devl = [LayerTensors(dev_t(h["Q"], tdt), dev_t(h["K"], tdt), dev_t(h["V"], tdt), dev_t(h["Wo"].T, tdt))
            for h in hostl]
    return hostl, devl


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_tiny_fp32_one_shot_step(dash, seed):
    """S=512, 4/4 heads, D=64, hidden 256, fp32: halt layer + top 50% + one post-halt layer (kv active)."""
    from attention_delta_token_amd.stack import OneShotStack
    w = WORKLOADS[0]
    hostl, devl = _stack_inputs(w, seed, "f32")
    say("tiny fp32 step seed", seed)
    k = oracle.topk_count(w.S, w.keep)
    st = OneShotStack(devl, halt_layer=0, keep=w.keep)
    assert st.k == k
    st.run()
    torch.cuda.synchronize()
    O_ref, U_ref, s_ref = oracle.attention_layer(hostl[0]["Q"], hostl[0]["K"], hostl[0]["V"], hostl[0]["Wo"])
    assert maxrel(host(st.U), U_ref) <= TOL_F32
    score = host(st.score)
    assert np.all(np.abs(score - s_ref) <= TOL_SCORE * s_ref)
    idx = st.idx.cpu().numpy()
    np.testing.assert_array_equal(idx, oracle.select_topk(score, k))
    selection_within_cut(idx, s_ref, k)
    Oa = oracle.attn_active(hostl[1]["Q"], hostl[1]["K"], hostl[1]["V"], idx, "active")
    Ua = oracle.output_projection(Oa, hostl[1]["Wo"])
    assert maxrel(host(st.Oa), Oa) <= TOL_F32
    assert maxrel(host(st.Ua), Ua) <= TOL_F32


def test_tiny_fp32_one_shot_step_forced(dash):
    """As above with the pages' forced retention (first 64, last 32 tokens) and
    K_eff = 96 + floor(0.5 * (512 - 96)) = 304."""
    from attention_delta_token_amd.stack import OneShotStack
    w = WORKLOADS[0]
    hostl, devl = _stack_inputs(w, 0, "f32")
    k = oracle.effective_keep_count(w.S, w.keep, 64, 32)
    assert k == 304
    st = OneShotStack(devl, halt_layer=0, keep=w.keep, keep_first=64, keep_last=32)
    assert st.k == k
    st.run()
    torch.cuda.synchronize()
    score, idx = host(st.score), st.idx.cpu().numpy()
    np.testing.assert_array_equal(idx, oracle.select_topk_forced(score, k, 64, 32))
    assert np.all(idx[:64] == np.arange(64)) and np.all(idx[-32:] == np.arange(w.S - 32, w.S))
    Oa = oracle.attn_active(hostl[1]["Q"], hostl[1]["K"], hostl[1]["V"], idx, "active")
    Ua = oracle.output_projection(Oa, hostl[1]["Wo"])
    assert maxrel(host(st.Ua), Ua) <= TOL_F32


@pytest.mark.parametrize("dtype,mode", [("f32", "active"), ("f32", "all"), ("bf16", "active")])
def test_multi_shot_stack(dash, dtype, mode):
    """Two halting decisions (layers 0 and 2 of 4): each decision bit-exact against
    the oracle's top-k of the GPU's own scores, the scores and the last layer
    against the oracle teacher-forced on the GPU's position sets."""
    from attention_delta_token_amd.stack import MultiShotStack
    w = WORKLOADS[0].scaled(layers=4) if dtype == "f32" else WORKLOADS[1].scaled(S=1024, hidden=512, layers=4)
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    tol = TOL_F32 if dtype == "f32" else TOL_BF16
    k1, k2 = (3 * w.S) // 4, (3 * w.S) // 10
    hostl, devl = _stack_inputs(w, 0, dtype)
    say("multi-shot", dtype, mode, w.S, k1, k2)
    st = MultiShotStack(devl, [(0, k1), (2, k2)], kv_mode=dash.DASH_KV_ACTIVE if mode == "active" else dash.DASH_KV_ALL)
    st.keep_scores = True
    st.run()
    torch.cuda.synchronize()
    (l1, p1, s0), (l2, p2, s2) = st.record
    idx1, idx2 = p1.cpu().numpy(), p2.cpu().numpy()
    s0, s2 = host(s0), host(s2)
    x0 = hostl[0]
    _, _, s0_ref = oracle.attention_layer(x0["Q"], x0["K"], x0["V"], x0["Wo"])
    assert np.all(np.abs(s0 - s0_ref) <= TOL_SCORE * s0_ref)
    np.testing.assert_array_equal(idx1, oracle.select_topk(s0, k1))
    x2 = hostl[2]
    s2_ref = oracle.delta_attn(oracle.output_projection(oracle.attn_active(x2["Q"], x2["K"], x2["V"], idx1, mode),
                                                        x2["Wo"]))
    assert np.all(np.abs(s2 - s2_ref) <= TOL_SCORE * s2_ref)
    np.testing.assert_array_equal(idx2, idx1[oracle.select_topk(s2, k2)])
    x3 = hostl[3]
    U3 = oracle.output_projection(oracle.attn_active(x3["Q"], x3["K"], x3["V"], idx2, mode), x3["Wo"])
    assert maxrel(host(st.Ua)[:k2], U3) <= tol


# ---------------------------------------------------------------------------
# decode over the pruned KV cache
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("S,n_new,mode,Hq,Hkv,D", [(900, 1, "active", 28, 4, 128), (900, 4, "active", 28, 4, 128),
                                                   (700, 2, "all", 8, 2, 64), (8192, 1, "active", 28, 4, 128),
                                                   (3000, 3, "all", 32, 8, 128), (600, 5, "all", 12, 2, 64),
                                                   (70000, 1, "active", 8, 2, 64)])
def test_decode_vs_oracle(dash, S, n_new, mode, Hq, Hkv, D):
    """B = 2 samples: the cache holds each sample's kept prefill rows (kv active) or
    all of them (kv all), then the new tokens' own K/V; every new token against the
    oracle's decode step.  The cases span 6 to 30 rows per kv-head (g * n_new) and,
    at S = 70000, caches long enough that each wave takes several 64-key steps."""
    B = 2
    w = WORKLOADS[1].scaled(S=S, Hq=Hq, Hkv=Hkv, D=D, hidden=Hq * D)
    pre = [layer_inputs(w, 70 + b, 0) for b in range(B)]
    new = [layer_inputs(w.scaled(S=n_new), 80 + b, 0) for b in range(B)]
    rng = np.random.default_rng(S + n_new)
    idx = [np.sort(rng.choice(S, int(S * (0.5 - 0.1 * b)), replace=False)) if mode == "active" else np.arange(S)
           for b in range(B)]
    cap = S + n_new
    Kc = np.zeros((B, cap, Hkv, D), np.float32)
    Vc = np.zeros((B, cap, Hkv, D), np.float32)
    n_kv = []
    for b in range(B):
        m = len(idx[b])
        Kc[b, :m], Vc[b, :m] = pre[b]["K"][idx[b]], pre[b]["V"][idx[b]]
        Kc[b, m:m + n_new], Vc[b, m:m + n_new] = new[b]["K"], new[b]["V"]
        n_kv.append(m + n_new)
    Qd = dev_t(np.stack([x["Q"] for x in new]))
    Od = torch.zeros(B, n_new, Hq * D, device="cuda", dtype=torch.bfloat16)
    say("decode", S, n_new, mode, Hq, Hkv, D, n_kv)
    dash.dash_decode(Qd, dev_t(Kc), dev_t(Vc), torch.tensor(n_kv, dtype=torch.int32, device="cuda"), Od)
    torch.cuda.synchronize()
    for b in range(B):
        ref = oracle.decode_step(new[b]["Q"], new[b]["K"], new[b]["V"], pre[b]["K"], pre[b]["V"], idx[b], mode)
        assert maxrel(host(Od)[b], ref) <= TOL_BF16


@pytest.mark.parametrize("D", [128, 64])
def test_decode_ignores_rows_past_the_count(dash, D):
    """Cache rows at or past a sample's count may hold anything (here NaN and
    infinities in K and V): the output equals the one over a clean cache."""
    B, S, n_new, Hq, Hkv = 2, 3000, 2, 14, 2
    w = WORKLOADS[1].scaled(S=S, Hq=Hq, Hkv=Hkv, D=D, hidden=Hq * D)
    x = [layer_inputs(w, 90 + b, 0) for b in range(B)]
    n_kv = [1700, 2333]
    Kc = np.zeros((B, S, Hkv, D), np.float32)
    Vc = np.zeros((B, S, Hkv, D), np.float32)
    for b in range(B):
        Kc[b, :n_kv[b]], Vc[b, :n_kv[b]] = x[b]["K"][:n_kv[b]], x[b]["V"][:n_kv[b]]
    Qd = dev_t(np.stack([x[b]["Q"][n_kv[b] - n_new:n_kv[b]] for b in range(B)]))
    nk = torch.tensor(n_kv, dtype=torch.int32, device="cuda")
    say("decode rows past the count", D)
    clean = torch.zeros(B, n_new, Hq * D, device="cuda", dtype=torch.bfloat16)
    dash.dash_decode(Qd, dev_t(Kc), dev_t(Vc), nk, clean)
    for b in range(B):
        Kc[b, n_kv[b]:] = np.nan
        Vc[b, n_kv[b]:] = np.inf
        Kc[b, n_kv[b]::7] = -np.inf
    dirty = torch.zeros(B, n_new, Hq * D, device="cuda", dtype=torch.bfloat16)
    dash.dash_decode(Qd, dev_t(Kc), dev_t(Vc), nk, dirty)
    torch.cuda.synchronize()
    assert torch.equal(clean, dirty)
    assert bool(torch.isfinite(clean.float()).all())


def test_decode_graph_replay(dash):
    """Decode calls captured in a HIP graph: every replay, with eager work and
    synchronisations in between, gives the eager call's output bit for bit (the
    library records no memsets, so nothing in the graph depends on replay order)."""
    Hq, Hkv, D, rows = 28, 4, 128, 1500
    g = torch.Generator(device="cpu").manual_seed(11)
    Qd = torch.randn(1, 1, Hq, D, generator=g).to("cuda", torch.bfloat16)
    Kc = torch.randn(1, rows, Hkv, D, generator=g).to("cuda", torch.bfloat16)
    Vc = torch.randn(1, rows, Hkv, D, generator=g).to("cuda", torch.bfloat16)
    n_kv = torch.tensor([rows - 7], dtype=torch.int32, device="cuda")
    Od = torch.empty(1, 1, Hq * D, device="cuda", dtype=torch.bfloat16)
    ws = dash.workspace(dash.DASH_OP_DECODE, dash.make_shape(1, rows, Hq, Hkv, D, Hq * D, dash.DASH_BF16), 1)
    say("decode graph replay", rows)
    dash.dash_decode(Qd, Kc, Vc, n_kv, Od, ws=ws)
    torch.cuda.synchronize()
    ref = Od.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        dash.dash_decode(Qd, Kc, Vc, n_kv, Od, ws=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(3):
            dash.dash_decode(Qd, Kc, Vc, n_kv, Od, ws=ws)
    other = torch.empty_like(Od)
    for rep in range(4):
        Od.zero_()
        dash.dash_decode(Qd, Kc, Vc, torch.tensor([rows // 2], dtype=torch.int32, device="cuda"), other, ws=ws)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(Od, ref), rep


# ---------------------------------------------------------------------------
# ragged (packed) batches: every sample against the oracle on its own slice
# ---------------------------------------------------------------------------

def _packed_layer(lengths, Hq, Hkv, D, hidden, dtype, seed, layer=0):
    """Per-sample seeded inputs packed back to back; W_o shared (the first sample's)."""
    xs = [layer_inputs(WORKLOADS[1].scaled(S=n, Hq=Hq, Hkv=Hkv, D=D, hidden=hidden, dtype=dtype), seed + b, layer)
          for b, n in enumerate(lengths)]
    cat = {n: np.concatenate([x[n] for x in xs]) for n in ("Q", "K", "V")}
    cat["Wo"] = xs[0]["Wo"]
    return xs, cat


def _cu(lengths):
    return np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_attn_layer_varlen(dash, dtype):
    lengths = [300, 77, 1, 513, 128]
    Hq, Hkv, D, hidden = 8, 2, (128 if dtype == "bf16" else 64), 256
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    xs, cat = _packed_layer(lengths, Hq, Hkv, D, hidden, dtype, seed=40)
    T = sum(lengths)
    cu = _cu(lengths)
    Q, K, V = (dev_t(cat[n], tdt) for n in ("Q", "K", "V"))
    Wo = dev_t(cat["Wo"].T, tdt)
    O = torch.empty(T, Hq * D, device="cuda", dtype=tdt)
    U = torch.empty(T, hidden, device="cuda", dtype=tdt)
    sc = torch.empty(T, device="cuda", dtype=torch.float32)
    dc = dash.DASH_BF16 if dtype == "bf16" else dash.DASH_F32
    ws = dash.workspace(dash.DASH_OP_ATTN_LAYER, dash.make_shape(1, T, Hq, Hkv, D, hidden, dc), T)
    say("attn layer varlen", dtype, lengths)
    dash.dash_attn_layer_varlen(Q, K, V, Wo, O, U, torch.from_numpy(cu).cuda(), max(lengths), sc, ws)
    torch.cuda.synchronize()
    for b, x in enumerate(xs):
        sl = slice(cu[b], cu[b + 1])
        O_ref, U_ref, s_ref = oracle.attention_layer(x["Q"], x["K"], x["V"], cat["Wo"])
        assert maxrel(host(O)[sl], O_ref) <= tol
        assert maxrel(host(U)[sl], U_ref) <= tol
        assert np.all(np.abs(host(sc)[sl] - s_ref) <= TOL_SCORE * s_ref)


def test_select_ragged_bit_exact(dash):
    lengths = [1000, 1, 37, 8192, 5000, 70000, 4]
    rng = np.random.default_rng(5)
    s = np.concatenate([score_vector(["normal", "equal", "bf16ties", "fewvalues", "perm", "normal", "special"][b],
                                     n, seed=b) for b, n in enumerate(lengths)])
    cu = _cu(lengths)
    for f, l in ((0, 0), (3, 2)):
        ks = [min(n, max(f + l, int(rng.integers(0, n + 1)))) for n in lengths]
        ks[1] = 1 if f + l == 0 else ks[1]
        cuk = _cu(ks)
        idx = torch.full((int(cuk[-1]),), -5, dtype=torch.int32, device="cuda")
        say("select ragged", lengths, ks, f, l)
        dash.dash_select_ragged(torch.from_numpy(s).cuda(), idx, torch.from_numpy(cu).cuda(),
                                torch.from_numpy(cuk).cuda(), max(lengths), keep_first=f, keep_last=l)
        torch.cuda.synchronize()
        got = idx.cpu().numpy()
        for b, n in enumerate(lengths):
            fb = min(f, ks[b])
            lb = min(l, ks[b] - fb)
            ref = oracle.select_topk_forced(s[cu[b]:cu[b + 1]], ks[b], fb, lb) + cu[b]
            np.testing.assert_array_equal(got[cuk[b]:cuk[b + 1]], ref)


@pytest.mark.parametrize("dtype,mode", [("bf16", "active"), ("bf16", "all"), ("f32", "active")])
def test_ragged_one_shot_step(dash, dtype, mode):
    """Packed samples of different lengths, each keeping its own share: the halting
    layer and each sample's selection (bit-exact on the GPU's scores) and the
    post-halt layer teacher-forced, all per sample against the oracle."""
    from attention_delta_token_amd.stack import LayerTensors, RaggedOneShotStack
    lengths = [700, 256, 1024, 90, 1]
    Hq, Hkv, D, hidden = 8, 2, (128 if dtype == "bf16" else 64), 384
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    packs = [_packed_layer(lengths, Hq, Hkv, D, hidden, dtype, seed=60, layer=l) for l in range(2)]
    layers = [LayerTensors(*(dev_t(c[n], tdt) for n in ("Q", "K", "V")), dev_t(c["Wo"].T, tdt)) for _, c in packs]
    st = RaggedOneShotStack(layers, lengths, halt_layer=0, keep=0.4,
                            kv_mode=dash.DASH_KV_ACTIVE if mode == "active" else dash.DASH_KV_ALL)
    say("ragged one-shot", dtype, mode, lengths, st.ks)
    st.run()
    torch.cuda.synchronize()
    cu, cuk = _cu(lengths), _cu(st.ks)
    score, idx = host(st.score), st.idx.cpu().numpy()
    (xs0, c0), (xs1, c1) = packs
    for b, n in enumerate(lengths):
        sl = slice(cu[b], cu[b + 1])
        _, U_ref, s_ref = oracle.attention_layer(xs0[b]["Q"], xs0[b]["K"], xs0[b]["V"], c0["Wo"])
        assert maxrel(host(st.U)[sl], U_ref) <= tol
        assert np.all(np.abs(score[sl] - s_ref) <= TOL_SCORE * s_ref)
        mine = idx[cuk[b]:cuk[b + 1]] - cu[b]
        np.testing.assert_array_equal(mine, oracle.select_topk(score[sl], st.ks[b]))
        if st.ks[b] == 0:  # nothing kept (the one-token sample at keep 0.4)
            continue
        Oa = oracle.attn_active(xs1[b]["Q"], xs1[b]["K"], xs1[b]["V"], mine, mode)
        assert maxrel(host(st.Ua)[cuk[b]:cuk[b + 1]], oracle.output_projection(Oa, c1["Wo"])) <= tol


@pytest.mark.timeout(900)
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_qwen_s8192_one_shot_step(dash, seed):
    """S=8192, 28/4 heads, D=128, hidden 3584, bf16: the full halt layer against the oracle,
    the selection bit-exact on the GPU scores and within the cut band on the oracle's,
    the post-halt layer teacher-forced on the GPU's active set."""
    from attention_delta_token_amd.stack import OneShotStack
    w = WORKLOADS[1]
    hostl, devl = _stack_inputs(w, seed, "bf16")
    say("qwen s8192 step seed", seed)
    k = oracle.topk_count(w.S, w.keep)
    st = OneShotStack(devl, halt_layer=0, keep=w.keep)
    assert st.k == k
    st.run()
    torch.cuda.synchronize()
    score, idx = host(st.score), st.idx.cpu().numpy()
    U = host(st.U)
    O_ref, U_ref, s_ref = oracle.attention_layer(hostl[0]["Q"], hostl[0]["K"], hostl[0]["V"], hostl[0]["Wo"])
    assert maxrel(host(st.O), O_ref) <= TOL_BF16
    assert maxrel(U, U_ref) <= TOL_BF16
    assert np.all(np.abs(score - s_ref) <= TOL_SCORE * s_ref)
    np.testing.assert_array_equal(idx, oracle.select_topk(score, k))
    nd = selection_within_cut(idx, s_ref, k)
    say("qwen s8192: tokens differing from the oracle selection:", nd)
    Oa = oracle.attn_active(hostl[1]["Q"], hostl[1]["K"], hostl[1]["V"], idx, "active")
    Ua = oracle.output_projection(Oa, hostl[1]["Wo"])
    assert maxrel(host(st.Oa), Oa) <= TOL_BF16
    assert maxrel(host(st.Ua), Ua) <= TOL_BF16
    # determinism: a second run reproduces every bit
    U1, s1, i1, Ua1 = st.U.clone(), st.score.clone(), st.idx.clone(), st.Ua.clone()
    st.run()
    torch.cuda.synchronize()
    assert torch.equal(U1, st.U) and torch.equal(s1, st.score) and torch.equal(i1, st.idx)
    assert torch.equal(Ua1, st.Ua)


def test_trace_select_records_only_chosen_kinds(dash):
    """dash_trace_select limits the event pairs to the chosen launch kinds (the
    bench brackets only attention launches inside its timed steps)."""
    x = _layer(300, 8, 2, 128, 256, seed=3)
    say("trace select")
    dash.trace_start(16)
    dash.trace_select(("attn_layer",))
    _run_layer(dash, x)
    dash.trace_stop()
    recs = dash.trace_read(16)
    assert [op for op, _ in recs] == ["attn_layer"]
    assert recs[0][1] > 0.0
    dash.trace_start(16)  # a new start records every kind again
    _run_layer(dash, x)
    dash.trace_stop()
    assert [op for op, _ in dash.trace_read(16)] == ["attn_layer", "proj_layer"]
