"""Whole-stack parity on the GPU for the stacks the long workloads define,
run through the stack drivers themselves:

* S=32768, Qwen2.5-7B shapes, 28 layers, one-shot halt at layer 11, keep 0.5,
  kv active (seeds 0-2);
* S=131072, same shapes, clustered salience, 28 layers, halt at 11, keep 0.3
  (seed 0);
* S=65536, Llama-3.1-8B shapes, 32 layers, threshold halting (30th
  percentile of the layer-0 scores, patience 2), kv all (seed 0);
* a reduced threshold stack (S=1536) checked in full over seeds 0-2.

Protocol (so that differences do not cascade):
* The decisions are bit-exact against the oracle fed the GPU's own scores
  (top-k, order statistic, every threshold step).
* End-to-end, a token may sit on different sides of the cut on the GPU and in
  the oracle only if its oracle score lies within 1e-2 relative of the
  oracle's cut (the k-th largest oracle score; for the threshold stack the
  oracle's tau).  At S=32768 the halting layer is checked in full (O, U and
  every score).  At S=131072 and at the threshold stack's layer 0 the oracle
  scores every token whose GPU score lies within 3e-2 of the GPU's cut, plus
  512 sampled rows: tokens outside that band keep their side of the cut as
  long as their scores are within the 1e-2 tolerance (checked on the
  samples), so the oracle's cut is fixed by the band alone.
* Post-halt layers are teacher-forced on the GPU's active set: 512 sampled
  rows per layer (always the first and last active row), the first post-halt
  layer in full at S=32768 and on 4096 rows at S=131072.
Tolerances: O and U max|Δ| <= 2e-2 * max|ref| (the maximum over the rows
compared), Δattn |Δ| <= 1e-2 * ref per token.
"""
import time

import numpy as np
import pytest
import torch

import oracle
import oracle_par
from workload import WORKLOADS, layer_inputs

pytestmark = pytest.mark.gpu

TOL_BF16 = 2e-2
TOL_SCORE = 1e-2
BAND = 3e-2  # relative band of GPU scores around the GPU's cut that the oracle scores in full


@pytest.fixture(scope="module")
def dash():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import attention_delta_token_amd as d
    d.load()
    return d


T0 = time.time()


def say(*a):
    print(f"[{time.time() - T0:7.1f}s]", *a, flush=True)


def dev_t(a, dtype=torch.bfloat16):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda", dtype)


def host(t):
    return t.float().cpu().numpy() if t.dtype == torch.bfloat16 else t.cpu().numpy()


def maxrel(got, ref):
    return float(np.max(np.abs(np.asarray(got, np.float64) - ref)) / np.max(np.abs(ref)))


def upload(h):
    from attention_delta_token_amd.stack import LayerTensors
    return LayerTensors(dev_t(h["Q"]), dev_t(h["K"]), dev_t(h["V"]), dev_t(h["Wo"].T))


def upload_stack(w, seed):
    layers = []
    for l in range(w.layers):
        layers.append(upload(layer_inputs(w, seed, l)))
    say(f"{w.name}: {w.layers} layers uploaded (seed {seed})")
    return layers


def sample_rows(n, count, seed):
    rng = np.random.default_rng(seed)
    rows = rng.choice(n, min(n, count), replace=False)
    return np.unique(np.concatenate([rows, [0, n - 1]])).astype(np.int64)


def rows_of(t, rows):
    """Rows of a device tensor, gathered on the device, as a host array."""
    return host(t[torch.from_numpy(np.asarray(rows, dtype=np.int64)).cuda()])


def check_scores(s_gpu, s_ref):
    bad = np.abs(s_gpu - s_ref) > TOL_SCORE * s_ref
    assert not np.any(bad), (np.nonzero(bad)[0][:10], s_gpu[bad][:10], s_ref[bad][:10])


def topk_band_check(x, s_g, k, gpu_idx, seed, O_dev, U_dev):
    """Oracle scores for every token within BAND of the GPU's cut plus 512
    sampled rows; the oracle's cut follows from them (see the module notes).
    Returns (oracle cut, tokens on different sides, tokens in the band)."""
    S = s_g.shape[0]
    s64 = s_g.astype(np.float64)
    c_g = np.sort(s64)[::-1][k - 1]
    near = np.nonzero(np.abs(s64 - c_g) <= BAND * c_g)[0]
    samp = sample_rows(S, 512, seed)
    rows = np.union1d(near, samp)
    say(f"band: {near.size} tokens within {BAND} of the GPU cut; oracle on {rows.size} rows")
    O_r, U_r, s_r = oracle_par.layer_rows(x, rows)
    check_scores(s64[rows], s_r)
    at = np.searchsorted(rows, samp)
    assert maxrel(rows_of(O_dev, samp), O_r[at]) <= TOL_BF16
    assert maxrel(rows_of(U_dev, samp), U_r[at]) <= TOL_BF16
    r_near = s_r[np.searchsorted(rows, near)]
    R_hi = c_g * (1 + BAND) / (1 + TOL_SCORE)  # every token above the band has an oracle score above this
    R_lo = c_g * (1 - BAND) / (1 - TOL_SCORE)  # ... and every token below it one below this
    above = int(np.sum(s64 > c_g * (1 + BAND)))
    hi = r_near > R_hi
    mid = np.nonzero((r_near >= R_lo) & ~hi)[0]
    need = k - above - int(hi.sum())
    assert 1 <= need <= mid.size, "the oracle's cut lies outside the band"
    mid_order = mid[np.lexsort((near[mid], -r_near[mid]))]  # larger score first, ties to the lower position
    cut_r = r_near[mid_order[need - 1]]
    ref_set = np.union1d(near[hi], near[mid_order[:need]])
    gpu_set = np.intersect1d(gpu_idx, near)
    diff = np.setxor1d(ref_set, gpu_set)
    r_diff = r_near[np.searchsorted(near, diff)]
    assert np.all(np.abs(r_diff - cut_r) <= TOL_SCORE * cut_r), (diff[:10], r_diff[:10], cut_r)
    return cut_r, int(diff.size), int(near.size)


# ---------------------------------------------------------------------------
# one-shot stacks: 28 layers, halt at layer 11
# ---------------------------------------------------------------------------

def _run_one_shot(dash, w, seed):
    from attention_delta_token_amd.stack import OneShotStack
    layers = upload_stack(w, seed)
    k = oracle.topk_count(w.S, w.keep)
    st = OneShotStack(layers, halt_layer=w.halt_layer, keep=w.keep)
    assert st.k == k
    st.record_post = True
    st.run()
    torch.cuda.synchronize()
    say(f"{w.name}: stack ran (k={k})")
    assert int(st.status[0].item()) == 0  # no NaN score at the decision
    return st, k


def _check_post_layers(w, seed, st, idx, first_rows):
    """Teacher-forced post-halt layers: queries at the GPU's kept positions, keys
    and values at the same positions (kv active)."""
    k = idx.shape[0]
    for n_l, (l, Oa_d, Ua_d) in enumerate(st.trace):
        x = layer_inputs(w, seed, l)
        sel = np.arange(k) if (n_l == 0 and first_rows >= k) else sample_rows(
            k, first_rows if n_l == 0 else 512, 1000 * seed + l)
        O_r, U_r, _ = oracle_par.layer_rows(x, idx[sel], kv_rows=idx)
        eo, eu = maxrel(rows_of(Oa_d, sel), O_r), maxrel(rows_of(Ua_d, sel), U_r)
        say(f"post-halt layer {l}: {sel.size} rows, O err {eo:.2e}, U err {eu:.2e}")
        assert eo <= TOL_BF16 and eu <= TOL_BF16
        del x


@pytest.mark.timeout(900)
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_qwen28_s32768_stack(dash, seed):
    """S=32768, 28 layers, halt at 11, keep 0.5: the halting layer in full, the
    selection against the oracle's own cut, every post-halt layer."""
    w = WORKLOADS[2]
    st, k = _run_one_shot(dash, w, seed)
    score, idx = host(st.score), st.idx.cpu().numpy()
    np.testing.assert_array_equal(idx, oracle.select_topk(score, k))  # bit-exact on the GPU's scores
    x = layer_inputs(w, seed, w.halt_layer)
    O_r, U_r, s_r = oracle_par.layer_rows(x, np.arange(w.S))
    say("halting layer: oracle done")
    eo, eu = maxrel(host(st.O), O_r), maxrel(host(st.U), U_r)
    say(f"halting layer: O err {eo:.2e}, U err {eu:.2e}")
    assert eo <= TOL_BF16 and eu <= TOL_BF16
    check_scores(score.astype(np.float64), s_r)
    ref_idx = oracle.select_topk(s_r, k)
    diff = np.setxor1d(idx, ref_idx)
    cut = np.sort(s_r)[::-1][k - 1]
    assert np.all(np.abs(s_r[diff] - cut) <= TOL_SCORE * cut)
    say(f"selection: {diff.size} tokens on different sides of the oracle's cut (all within 1e-2 of it)")
    del O_r, U_r, x
    _check_post_layers(w, seed, st, idx, first_rows=k)


@pytest.mark.timeout(900)
def test_qwen28clust_s131072_stack(dash):
    """S=131072 clustered, 28 layers, halt at 11, keep 0.3 (k = 39321)."""
    w = WORKLOADS[4]
    seed = 0
    st, k = _run_one_shot(dash, w, seed)
    score, idx = host(st.score), st.idx.cpu().numpy()
    assert k == 39321 and idx.shape[0] == k
    np.testing.assert_array_equal(idx, oracle.select_topk(score, k))
    x = layer_inputs(w, seed, w.halt_layer)
    cut_r, nd, nb = topk_band_check(x, score, k, idx, seed, st.O, st.U)
    say(f"selection: oracle cut {cut_r:.6g}; {nd} of {nb} band tokens on different sides (all within 1e-2)")
    del x
    from workload import span_slots
    in_span = np.zeros(w.S, bool)
    for s0 in span_slots(w, seed):
        in_span[s0:s0 + 256] = True
    say("kept fraction inside the salient spans", float(in_span[idx].mean()),
        "outside", float((~in_span[idx]).sum() / (~in_span).sum()))
    _check_post_layers(w, seed, st, idx, first_rows=4096)


# ---------------------------------------------------------------------------
# threshold stacks (kv all)
# ---------------------------------------------------------------------------

def _check_threshold_stack(dash, w, seed, full):
    """full: every row of every layer against the oracle (small S).  Otherwise
    the band protocol at layer 0 and 512 sampled active rows per later layer."""
    from attention_delta_token_amd.stack import ThresholdStack
    layers = upload_stack(w, seed)
    rank = oracle.percentile_rank(w.S, w.tau_pct)
    st = ThresholdStack(layers, tau_pct=w.tau_pct, patience=w.patience, record=True)
    assert st.rank == rank
    st.run()
    torch.cuda.synchronize()
    say(f"{w.name}: threshold stack ran")
    S = w.S
    score0 = host(st.trace[0][1])
    tau = float(st.tau[0].item())
    # tau: bit-exact order statistic of the GPU's own layer-0 scores
    assert np.float32(tau) == np.float32(oracle.order_statistic(score0, rank))
    x0 = layer_inputs(w, seed, 0)
    s64 = score0.astype(np.float64)
    if full:
        _, U_r, s_r = oracle_par.layer_rows(x0, np.arange(S))
        check_scores(s64, s_r)
        tau_ref = oracle.order_statistic(s_r, rank)
        ref_below = s_r < tau_ref
        gpu_below = score0 < tau
        diff = np.nonzero(ref_below != gpu_below)[0]
        assert np.all(np.abs(s_r[diff] - tau_ref) <= TOL_SCORE * tau_ref)
    else:
        near = np.nonzero(np.abs(s64 - tau) <= BAND * tau)[0]
        samp = sample_rows(S, 512, seed)
        rows = np.union1d(near, samp)
        say(f"layer 0: {near.size} tokens within {BAND} of the GPU's tau; oracle on {rows.size} rows")
        _, U_r, s_r = oracle_par.layer_rows(x0, rows)
        check_scores(s64[rows], s_r)
        r_near = s_r[np.searchsorted(rows, near)]
        R_lo = tau * (1 - BAND) / (1 - TOL_SCORE)
        R_hi = tau * (1 + BAND) / (1 + TOL_SCORE)
        below = int(np.sum(s64 < tau * (1 - BAND)))
        lo = r_near < R_lo
        mid = np.sort(r_near[(r_near >= R_lo) & (r_near <= R_hi)])
        need = rank - below - int(lo.sum())
        assert 1 <= need <= mid.size, "the oracle's tau lies outside the band"
        tau_ref = float(mid[need - 1])
        gpu_below = score0[near] < tau
        ref_below = r_near < tau_ref
        d = ref_below != gpu_below
        assert np.all(np.abs(r_near[d] - tau_ref) <= TOL_SCORE * tau_ref)
    say(f"tau: GPU {tau:.6g}, oracle {tau_ref:.6g}")
    assert abs(tau - tau_ref) <= TOL_SCORE * tau_ref
    del x0
    # every later layer: decisions replayed bit-exact on the GPU scores, outputs teacher-forced
    pos_h = np.arange(S, dtype=np.int32)
    cnt_h = np.zeros(S, dtype=np.uint8)
    pos_h, cnt_h = oracle.threshold_step(score0, pos_h, cnt_h, tau, w.patience)
    active = [S, pos_h.shape[0]]
    for l in range(1, w.layers):
        pos_d, n_d, s_d, U_d = st.trace[l]
        n = int(n_d[0].item())
        pos_g = pos_d.cpu().numpy()[:n]
        np.testing.assert_array_equal(pos_g, pos_h)  # the active set the GPU used = the oracle's decisions
        s_g = host(s_d)[:n]
        sel = np.arange(n) if full else (sample_rows(n, 512, 1000 * seed + l) if n > 0 else np.zeros(0, np.int64))
        if sel.size:
            x = layer_inputs(w, seed, l)
            _, Ua, sa = oracle_par.layer_rows(x, pos_g[sel])
            eu = maxrel(rows_of(U_d, sel), Ua)
            assert eu <= TOL_BF16
            check_scores(s_g[sel].astype(np.float64), sa)
            # a sampled token's side of tau differs from the oracle's only near the oracle's tau
            d = (s_g[sel] < tau) != (sa < tau_ref)
            assert np.all(np.abs(sa[d] - tau_ref) <= TOL_SCORE * tau_ref)
            if l % 8 == 0 or l == w.layers - 1:
                say(f"layer {l}: {n} active, {sel.size} rows checked, U err {eu:.2e}")
            del x
        pos_h, cnt_h = oracle.threshold_step(s_g, pos_h, cnt_h, tau, w.patience)
        active.append(pos_h.shape[0])
    m = int(st.n[st.final][0].item())
    np.testing.assert_array_equal(st.pos[st.final].cpu().numpy()[:m], pos_h)
    np.testing.assert_array_equal(st.counters.cpu().numpy(), cnt_h)
    assert int(st.status[0].item()) == 0  # no NaN score in the last threshold step
    say("active trajectory", active)
    return active


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_threshold_stack_reduced(dash, seed):
    """Llama-3.1-8B head shapes at S=1536, hidden 256, 6 layers, every row checked."""
    w = WORKLOADS[3].scaled(S=1536, hidden=256, layers=6)
    active = _check_threshold_stack(dash, w, seed, full=True)
    assert active[2] < w.S  # some tokens halt after two layers below tau


@pytest.mark.timeout(900)
def test_llama32_s65536_threshold_stack(dash):
    """S=65536, 32/8 heads, hidden 4096, all 32 layers."""
    w = WORKLOADS[3]
    active = _check_threshold_stack(dash, w, 0, full=False)
    assert len(active) == w.layers + 1 and active[-1] < w.S
