"""Whole-stack parity on the GPU: the threshold (selective-halting) stack with
full K/V, and the one-shot stacks at the full sequence lengths of the
Qwen2.5-7B / Llama-3.1-8B-shaped workloads.

Protocol (so that differences do not cascade): selection, order statistic and
threshold decisions are checked bit-exact against the oracle fed the GPU's own
scores; post-halt layers are teacher-forced on the GPU's active set; at full
length the oracle checks a seeded sample of rows (always including the first
and last row), which it can compute one by one.  Tolerances as in
test_gpu_parity.py.
"""
import numpy as np
import pytest
import torch

import oracle
from workload import WORKLOADS, layer_inputs

pytestmark = pytest.mark.gpu

TOL_BF16 = 2e-2
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
    return t.float().cpu().numpy() if t.dtype == torch.bfloat16 else t.cpu().numpy()


def maxrel(got, ref):
    return float(np.max(np.abs(np.asarray(got, np.float64) - ref)) / np.max(np.abs(ref)))


def upload(h):
    from attention_delta_token_amd.stack import LayerTensors
    return LayerTensors(dev_t(h["Q"]), dev_t(h["K"]), dev_t(h["V"]), dev_t(h["Wo"].T))


def sample_rows(n, count, seed):
    rng = np.random.default_rng(seed)
    rows = rng.choice(n, min(n, count), replace=False)
    return np.unique(np.concatenate([rows, [0, n - 1]])).astype(np.int64)


def sampled_layer_ref(x, rows):
    """Oracle O, U and score of the full-length layer for the given query rows."""
    O = oracle.causal_gqa_attention(x["Q"][rows], x["K"], x["V"], q_pos=rows)
    U = oracle.output_projection(O, x["Wo"])
    return O, U, oracle.delta_attn(U)


# ---------------------------------------------------------------------------
# threshold stack (kv all), reduced and full length
# ---------------------------------------------------------------------------

def _check_threshold_stack(dash, w, seed, full_rows_check):
    from attention_delta_token_amd.stack import ThresholdStack
    hostl = [layer_inputs(w, seed, l) for l in range(w.layers)]
    layers = [upload(h) for h in hostl]
    say("threshold stack", w.S, w.layers, "seed", seed)
    st = ThresholdStack(layers, tau_rank=w.tau_rank, patience=w.patience, record=True)
    st.run()
    torch.cuda.synchronize()
    S = w.S
    score0 = host(st.trace[0][1])
    tau = float(st.tau[0].item())
    # layer 0 against the oracle (full or sampled rows)
    if full_rows_check:
        _, U_ref, s_ref = oracle.attention_layer(hostl[0]["Q"], hostl[0]["K"], hostl[0]["V"], hostl[0]["Wo"])
        assert np.all(np.abs(score0 - s_ref) <= TOL_SCORE * s_ref)
        tau_ref = oracle.order_statistic(s_ref, w.tau_rank)
        assert abs(tau - tau_ref) <= TOL_SCORE * tau_ref
    else:
        rows = sample_rows(S, 96, seed)
        _, _, s_ref = sampled_layer_ref(hostl[0], rows)
        assert np.all(np.abs(score0[rows] - s_ref) <= TOL_SCORE * s_ref)
    # tau: bit-exact order statistic of the GPU's own layer-0 scores
    assert np.float32(tau) == np.float32(oracle.order_statistic(score0, w.tau_rank))
    pos_h = np.arange(S, dtype=np.int32)
    cnt_h = np.zeros(S, dtype=np.uint8)
    pos_h, cnt_h = oracle.threshold_step(score0, pos_h, cnt_h, tau, w.patience)
    active = [S, pos_h.shape[0]]
    for l in range(1, w.layers):
        pos_d, n_d, s_d, U_d = st.trace[l]
        n = int(n_d[0].item())
        pos_g = pos_d.cpu().numpy()[:n]
        np.testing.assert_array_equal(pos_g, pos_h)  # the active set the GPU used = oracle's decisions
        s_g = host(s_d)[:n]
        x = hostl[l]
        if full_rows_check:
            sel = np.arange(n)
        else:
            sel = sample_rows(n, 64, seed + l) if n > 0 else np.zeros(0, np.int64)
        if sel.size:
            Oa = oracle.causal_gqa_attention(x["Q"][pos_g[sel]], x["K"], x["V"], q_pos=pos_g[sel])
            Ua = oracle.output_projection(Oa, x["Wo"])
            sa = oracle.delta_attn(Ua)
            assert maxrel(host(U_d)[sel], Ua) <= TOL_BF16
            assert np.all(np.abs(s_g[sel] - sa) <= TOL_SCORE * sa)
        pos_h, cnt_h = oracle.threshold_step(s_g, pos_h, cnt_h, tau, w.patience)
        active.append(pos_h.shape[0])
    m = int(st.n[st.final][0].item())
    np.testing.assert_array_equal(st.pos[st.final].cpu().numpy()[:m], pos_h)
    np.testing.assert_array_equal(st.counters.cpu().numpy(), cnt_h)
    say("active trajectory", active)
    return active


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_threshold_stack_reduced(dash, seed):
    """Llama-3.1-8B head shapes at S=1536, hidden 256, 6 layers."""
    w = WORKLOADS[3].scaled(S=1536, hidden=256, layers=6)
    active = _check_threshold_stack(dash, w, seed, full_rows_check=True)
    assert active[2] < w.S  # some tokens halt after two layers below tau


@pytest.mark.timeout(1200)
def test_llama_s65536_threshold_stack(dash):
    """Full length S=65536, 32/8 heads, hidden 4096; 4 of the 32 layers (halting starts at layer 2)."""
    w = WORKLOADS[3].scaled(layers=4)
    active = _check_threshold_stack(dash, w, 0, full_rows_check=False)
    assert active[-1] < w.S


# ---------------------------------------------------------------------------
# one-shot stacks at full length: halt layer + first post-halt layer
# ---------------------------------------------------------------------------

@pytest.mark.timeout(1200)
@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("cfg", [2, 4])
def test_one_shot_full_length(dash, cfg, seed):
    """S=32768 (keep 0.5) and S=131072 clustered (keep 0.3): the halting layer at
    full length and the first post-halt layer (kv active)."""
    from attention_delta_token_amd.stack import OneShotStack
    w = WORKLOADS[cfg]
    hl = w.halt_layer
    hostl = [layer_inputs(w, seed, l) for l in (hl, hl + 1)]
    layers = [upload(h) for h in hostl]
    say("one-shot full length", w.name, w.S, "k", w.k, "seed", seed)
    st = OneShotStack(layers, halt_layer=0, k=w.k)
    st.run()
    torch.cuda.synchronize()
    score, idx = host(st.score), st.idx.cpu().numpy()
    assert idx.shape[0] == w.k
    # the selection is exactly the oracle's top-k of the GPU scores
    np.testing.assert_array_equal(idx, oracle.select_topk(score, w.k))
    # halt layer on sampled rows
    rows = sample_rows(w.S, 64, 10 * cfg + seed)
    O_ref, U_ref, s_ref = sampled_layer_ref(hostl[0], rows)
    assert maxrel(host(st.O)[rows], O_ref) <= TOL_BF16
    assert maxrel(host(st.U)[rows], U_ref) <= TOL_BF16
    assert np.all(np.abs(score[rows] - s_ref) <= TOL_SCORE * s_ref)
    # a sampled token differs from the oracle's choice only inside the cut band
    cut = np.sort(score)[::-1][w.k - 1]
    chosen = np.isin(rows, idx)
    # (the band is twice the score tolerance: GPU scores may sit 1e-2 off the oracle's)
    ref_chosen = s_ref >= cut * (1 + 2 * TOL_SCORE)
    ref_dropped = s_ref <= cut * (1 - 2 * TOL_SCORE)
    assert np.all(chosen[ref_chosen]) and not np.any(chosen[ref_dropped])
    # post-halt layer, teacher-forced on the GPU's active set
    x = hostl[1]
    sel = sample_rows(w.k, 64, 10 * cfg + seed + 7)
    Ka, Va = x["K"][idx], x["V"][idx]
    Oa = oracle.causal_gqa_attention(x["Q"][idx[sel]], Ka, Va, q_pos=sel)
    Ua = oracle.output_projection(Oa, x["Wo"])
    assert maxrel(host(st.Oa)[sel], Oa) <= TOL_BF16
    assert maxrel(host(st.Ua)[sel], Ua) <= TOL_BF16
    if w.clustered:
        from workload import span_slots
        spans = span_slots(w, seed)
        in_span = np.zeros(w.S, bool)
        for s0 in spans:
            in_span[s0:s0 + 256] = True
        say("clustered: kept fraction inside salient spans", float(in_span[idx].mean()),
            "outside", float((~in_span[idx]).sum() / (~in_span).sum()))
