"""Pins for the CPU oracle: each oracle function is checked against something
other than itself — brute force, closed forms, a library routine, hand-worked
fixtures under tests/golden/, and the method's own invariants.  CPU only."""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from workload import WORKLOADS, layer_inputs, score_vector, SCORE_KINDS, round_bf16


def _rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------

def brute_attention(Q, K, V, q_pos, kv_pos):
    """Double loop over (query, key) with explicit exp and sum, pure Python floats."""
    n_q, Hq, D = Q.shape
    n_kv, Hkv, _ = K.shape
    g = Hq // Hkv
    O = np.zeros((n_q, Hq * D))
    for h in range(Hq):
        j = h // g
        for i in range(n_q):
            keys = [r for r in range(n_kv) if kv_pos[r] <= q_pos[i]]
            logit = {}
            for r in keys:
                dot = 0.0
                for d in range(D):
                    dot += float(Q[i, h, d]) * float(K[r, j, d])
                logit[r] = dot / math.sqrt(D)
            mx = max(logit.values())
            w = {r: math.exp(logit[r] - mx) for r in keys}
            tot = sum(w.values())
            for d in range(D):
                acc = 0.0
                for r in keys:
                    acc += w[r] / tot * float(V[r, j, d])
                O[i, h * D + d] = acc
    return O


@pytest.mark.parametrize("Hq,Hkv", [(2, 2), (4, 2), (6, 3), (3, 1)])
def test_attention_brute_force(Hq, Hkv):
    g = _rng(Hq * 10 + Hkv)
    S, D = 9, 4
    Q = g.standard_normal((S, Hq, D)) * 2
    K = g.standard_normal((S, Hkv, D))
    V = g.standard_normal((S, Hkv, D))
    pos = np.arange(S)
    ref = brute_attention(Q, K, V, pos, pos)
    got = oracle.causal_gqa_attention(Q, K, V, block_rows=4)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_attention_brute_force_positions():
    g = _rng(7)
    Hq, Hkv, D = 4, 2, 3
    kv_pos = np.array([0, 2, 3, 7, 8, 11])
    q_pos = np.array([2, 7, 11])
    Q = g.standard_normal((3, Hq, D))
    K = g.standard_normal((6, Hkv, D))
    V = g.standard_normal((6, Hkv, D))
    ref = brute_attention(Q, K, V, q_pos, kv_pos)
    got = oracle.causal_gqa_attention(Q, K, V, q_pos=q_pos, kv_pos=kv_pos)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_attention_matches_torch_sdpa():
    """Library routine: torch's causal scaled-dot-product attention in float64 with GQA."""
    g = _rng(3)
    S, Hq, Hkv, D = 70, 8, 2, 16
    Q = g.standard_normal((S, Hq, D))
    K = g.standard_normal((S, Hkv, D))
    V = g.standard_normal((S, Hkv, D))
    q = torch.from_numpy(Q).permute(1, 0, 2)[None]
    k = torch.from_numpy(K).permute(1, 0, 2)[None]
    v = torch.from_numpy(V).permute(1, 0, 2)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True, enable_gqa=True)
    ref = ref[0].permute(1, 0, 2).reshape(S, Hq * D).numpy()
    got = oracle.causal_gqa_attention(Q, K, V, block_rows=32)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_attention_single_token_is_v0():
    g = _rng(1)
    Q = g.standard_normal((1, 4, 8))
    K = g.standard_normal((1, 2, 8))
    V = g.standard_normal((1, 2, 8))
    O = oracle.causal_gqa_attention(Q, K, V)
    for h in range(4):
        assert np.array_equal(O[0, h * 8:(h + 1) * 8], V[0, h // 2])


def test_attention_zero_query_is_prefix_mean_and_head_map():
    """Q = 0 gives uniform weights: O_i is the mean of V_0..V_i of kv-head h // g."""
    g = _rng(2)
    S, Hq, Hkv, D = 13, 6, 3, 5
    Q = np.zeros((S, Hq, D))
    K = g.standard_normal((S, Hkv, D))
    V = g.standard_normal((S, Hkv, D)) + np.arange(Hkv)[None, :, None] * 10.0
    O = oracle.causal_gqa_attention(Q, K, V, block_rows=5)
    for h in range(Hq):
        pm = np.cumsum(V[:, h // 2, :], axis=0) / np.arange(1, S + 1)[:, None]
        np.testing.assert_allclose(O[:, h * D:(h + 1) * D], pm, rtol=0, atol=1e-12)


def test_attention_dominant_diagonal_is_one_hot():
    S, D = 6, 8
    K = np.zeros((S, 1, D))
    Q = np.zeros((S, 1, D))
    for i in range(S):
        K[i, 0, i] = 1.0
        Q[i, 0, i] = 1000.0 * math.sqrt(D)
    V = _rng(4).standard_normal((S, 1, D))
    O = oracle.causal_gqa_attention(Q, K, V)
    np.testing.assert_allclose(O, V[:, 0, :], rtol=0, atol=1e-300)


def test_attention_scale_is_inv_sqrt_d():
    """Two keys with logits differing by a known amount: weights exp(Δ/√D) ratio."""
    D = 16
    Q = np.zeros((2, 1, D)); Q[1, 0, 0] = 2.0
    K = np.zeros((2, 1, D)); K[0, 0, 0] = 1.0; K[1, 0, 0] = 0.0
    V = np.zeros((2, 1, D)); V[0, 0, 1] = 1.0; V[1, 0, 1] = 0.0
    O = oracle.causal_gqa_attention(Q, K, V)
    a = math.exp(2.0 / math.sqrt(D))
    assert abs(O[1, 1] - a / (a + 1.0)) < 1e-15


# ---------------------------------------------------------------------------
# projection and score
# ---------------------------------------------------------------------------

def test_projection_brute_force_and_identity():
    g = _rng(5)
    O = g.standard_normal((4, 6))
    W = g.standard_normal((6, 3))
    U = oracle.output_projection(O, W)
    for t in range(4):
        for c in range(3):
            s = 0.0
            for e in range(6):
                s += O[t, e] * W[e, c]
            assert abs(U[t, c] - s) < 1e-12
    np.testing.assert_array_equal(oracle.output_projection(O, np.eye(6)), O)


def test_delta_attn_closed_forms(golden_dir):
    cases = json.load(open(os.path.join(golden_dir, "l2norm.json")))["cases"]
    for c in cases:
        assert oracle.delta_attn(np.array([c["row"]]))[0] == c["norm"]
    a, n = -1.25, 49
    assert oracle.delta_attn(np.full((1, n), a))[0] == pytest.approx(abs(a) * math.sqrt(n), rel=1e-15)
    row = np.zeros((1, 11)); row[0, 7] = -3.5
    assert oracle.delta_attn(row)[0] == 3.5


def test_attention_layer_score_is_norm_of_u():
    w = WORKLOADS[0].scaled(S=32)
    x = layer_inputs(w, 0, 0)
    O, U, s = oracle.attention_layer(x["Q"], x["K"], x["V"], x["Wo"])
    for t in (0, 5, 31):
        assert s[t] == pytest.approx(math.sqrt(sum(float(u) ** 2 for u in U[t])), rel=1e-14)
    np.testing.assert_allclose(U, O @ x["Wo"].astype(np.float64), rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# top-k selection
# ---------------------------------------------------------------------------

def _beats(a, b, i, j):
    """True when position j (score b) ranks ahead of position i (score a)."""
    an, bn = math.isnan(a), math.isnan(b)
    if bn and an:
        return j < i
    if bn:
        return False
    if an:
        return True
    if b > a:
        return True
    return b == a and j < i


def brute_topk(score, k):
    n = len(score)
    sel = []
    for i in range(n):
        rank = sum(1 for j in range(n) if j != i and _beats(float(score[i]), float(score[j]), i, j))
        if rank < k:
            sel.append(i)
    return np.array(sel, dtype=np.int32)


def test_topk_golden(golden_dir):
    for c in json.load(open(os.path.join(golden_dir, "topk_ties.json")))["cases"]:
        s = np.array([float(v) for v in c["score"]], dtype=np.float32)
        np.testing.assert_array_equal(oracle.select_topk(s, c["k"]), np.array(c["idx"], dtype=np.int32))


@pytest.mark.parametrize("kind", SCORE_KINDS)
@pytest.mark.parametrize("n", [1, 7, 64, 130])
def test_topk_brute_force(kind, n):
    s = score_vector(kind, n, seed=n)
    for k in sorted({0, 1, n // 3, n // 2, n - 1, n} & set(range(n + 1))):
        np.testing.assert_array_equal(oracle.select_topk(s, k), brute_topk(s, k))


def test_topk_special_orders():
    n = 100
    np.testing.assert_array_equal(oracle.select_topk(np.full(n, 3.0), 40), np.arange(40))
    np.testing.assert_array_equal(oracle.select_topk(np.linspace(1, 0, n), 40), np.arange(40))
    np.testing.assert_array_equal(oracle.select_topk(np.linspace(0, 1, n), 40), np.arange(60, 100))
    perm = _rng(9).permutation(n)
    got = oracle.select_topk(perm.astype(np.float64), 10)
    np.testing.assert_array_equal(got, np.sort(np.nonzero(perm >= n - 10)[0]))
    np.testing.assert_array_equal(oracle.select_topk(perm, n), np.arange(n))


def test_keep_counts(golden_dir):
    c = json.load(open(os.path.join(golden_dir, "counts.json")))
    for e in c["keep"]:
        assert oracle.topk_count(e["S"], e["keep"]) == e["k"]
    for e in c["rank"]:
        assert oracle.percentile_rank(e["S"], e["pct"]) == e["r"]
    # the workloads' own counts: S=131072 keep 0.3 truncates 39321.6; S=65536 30th percentile
    assert oracle.topk_count(WORKLOADS[4].S, WORKLOADS[4].keep) == 39321
    assert oracle.percentile_rank(WORKLOADS[3].S, WORKLOADS[3].tau_pct) == 19661


def brute_topk_forced(score, k, f, l):
    """Position i is kept iff it is one of the first f or last l, or it lies in
    the middle and fewer than k - f - l other middle positions beat it."""
    n = len(score)
    sel = []
    for i in range(n):
        if i < f or i >= n - l:
            sel.append(i)
            continue
        beaten_by = sum(1 for j in range(f, n - l)
                        if j != i and _beats(float(score[i]), float(score[j]), i, j))
        if beaten_by < k - f - l:
            sel.append(i)
    return np.array(sel, dtype=np.int32)


def test_forced_golden(golden_dir):
    for c in json.load(open(os.path.join(golden_dir, "topk_ties.json")))["forced_cases"]:
        s = np.array(c["score"], dtype=np.float32)
        got = oracle.select_topk_forced(s, c["k"], c["f"], c["l"])
        np.testing.assert_array_equal(got, np.array(c["idx"], dtype=np.int32))


def test_forced_counts(golden_dir):
    for e in json.load(open(os.path.join(golden_dir, "counts.json")))["forced"]:
        assert oracle.effective_keep_count(e["T"], e["keep"], e["f"], e["l"]) == e["k"]
    with pytest.raises(ValueError):
        oracle.effective_keep_count(10, 0.5, 6, 5)


@pytest.mark.parametrize("kind", SCORE_KINDS)
@pytest.mark.parametrize("n", [1, 9, 70])
def test_forced_brute_force(kind, n):
    s = score_vector(kind, n, seed=3 * n + 1)
    for f in sorted({0, 1, n // 4} & set(range(n + 1))):
        for l in sorted({0, 2, n // 5} & set(range(n - f + 1))):
            for k in sorted({f + l, f + l + 1, (n + f + l) // 2, n} & set(range(f + l, n + 1))):
                got = oracle.select_topk_forced(s, k, f, l)
                assert got.shape[0] == k
                np.testing.assert_array_equal(got, brute_topk_forced(s, k, f, l))


def test_forced_reduces_and_rejects():
    s = score_vector("normal", 50, seed=4)
    # no forced tokens: plain top-k; everything forced: the identity
    np.testing.assert_array_equal(oracle.select_topk_forced(s, 20, 0, 0), brute_topk(s, 20))
    np.testing.assert_array_equal(oracle.select_topk_forced(s, 50, 30, 20), np.arange(50))
    for bad in ((10, 6, 5), (60, 0, 0), (3, 2, 2), (5, -1, 0)):
        with pytest.raises(ValueError):
            oracle.select_topk_forced(s, *bad)


# ---------------------------------------------------------------------------
# order statistic
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("kind", SCORE_KINDS)
def test_order_statistic_brute_force(kind):
    n = 50
    s = score_vector(kind, n, seed=3)
    vals = [float(v) for v in s]
    nans = [v for v in vals if math.isnan(v)]
    rest = sorted(v for v in vals if not math.isnan(v))
    ordered = nans + rest
    for r in (1, 2, 15, 25, 49, 50):
        got = oracle.order_statistic(s, r)
        exp = ordered[r - 1]
        if math.isnan(exp):
            assert math.isnan(got)
        else:
            assert got == exp
            if exp == 0.0:
                assert math.copysign(1.0, got) == 1.0


# ---------------------------------------------------------------------------
# threshold halting
# ---------------------------------------------------------------------------

def test_threshold_golden(golden_dir):
    c = json.load(open(os.path.join(golden_dir, "threshold_sequences.json")))
    tau, pat = c["tau"], c["patience"]
    toks = c["tokens"]
    n, L = len(toks), len(toks[0]["scores"])
    seq = np.array([[float(v) for v in t["scores"]] for t in toks])
    counters = np.zeros(n, dtype=np.uint8)
    pos = np.arange(n, dtype=np.int32)
    halted_after = [None] * n
    for l in range(L):
        new_pos, counters = oracle.threshold_step(seq[pos, l], pos, counters, tau, pat)
        for p in set(pos.tolist()) - set(new_pos.tolist()):
            halted_after[p] = l
        pos = new_pos
    assert halted_after == [t["halt_after_layer"] for t in toks]


def test_threshold_step_leaves_inactive_counters():
    counters = np.array([5, 1, 0, 1], dtype=np.uint8)
    pos = np.array([1, 3], dtype=np.int32)
    new_pos, c2 = oracle.threshold_step(np.array([0.1, 0.9]), pos, counters, 0.5, 2)
    np.testing.assert_array_equal(new_pos, [3])
    np.testing.assert_array_equal(c2, [5, 2, 0, 0])


# ---------------------------------------------------------------------------
# compaction
# ---------------------------------------------------------------------------

def test_compact_explicit_loop():
    X = _rng(6).standard_normal((20, 3, 4))
    idx = np.array([0, 3, 4, 9, 19])
    got = oracle.compact(X, idx)
    for r, i in enumerate(idx):
        assert np.array_equal(got[r], X[i])
    assert oracle.compact(X, np.zeros(0, dtype=np.int32)).shape == (0, 3, 4)


# ---------------------------------------------------------------------------
# post-halt attention invariants
# ---------------------------------------------------------------------------

def _small_layer(S=40, Hq=4, Hkv=2, D=8, seed=0):
    g = _rng(seed)
    return (g.standard_normal((S, Hq, D)), g.standard_normal((S, Hkv, D)),
            g.standard_normal((S, Hkv, D)))


@pytest.mark.parametrize("mode", ["active", "all"])
def test_keep_all_is_dense(mode):
    Q, K, V = _small_layer()
    dense = oracle.causal_gqa_attention(Q, K, V)
    got = oracle.attn_active(Q, K, V, np.arange(40), mode)
    np.testing.assert_allclose(got, dense, rtol=0, atol=1e-12)


def test_kv_all_rows_equal_dense_rows():
    Q, K, V = _small_layer(seed=1)
    dense = oracle.causal_gqa_attention(Q, K, V)
    idx = np.sort(_rng(2).choice(40, 17, replace=False))
    got = oracle.attn_active(Q, K, V, idx, "all")
    np.testing.assert_allclose(got, dense[idx], rtol=0, atol=1e-12)


@pytest.mark.parametrize("mode", ["active", "all"])
def test_prefix_idx_is_dense_prefix(mode):
    Q, K, V = _small_layer(seed=3)
    dense = oracle.causal_gqa_attention(Q, K, V)
    got = oracle.attn_active(Q, K, V, np.arange(23), mode)
    np.testing.assert_allclose(got, dense[:23], rtol=0, atol=1e-12)


def test_kv_active_is_dense_on_compacted_sequence():
    Q, K, V = _small_layer(seed=4)
    idx = np.sort(_rng(5).choice(40, 15, replace=False))
    got = oracle.attn_active(Q, K, V, idx, "active")
    ref = brute_attention(Q[idx], K[idx], V[idx], np.arange(15), np.arange(15))
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# stacks
# ---------------------------------------------------------------------------

def test_one_shot_stack_keep_all_is_dense():
    w = WORKLOADS[0].scaled(S=48, layers=3, halt_layer=1)
    get = lambda l: layer_inputs(w, 0, l)
    res = oracle.run_one_shot(get, 3, 1, k=48)
    np.testing.assert_array_equal(res["idx"], np.arange(48))
    x = get(2)
    _, U, _ = oracle.attention_layer(x["Q"], x["K"], x["V"], x["Wo"])
    np.testing.assert_allclose(res["U"][2], U, rtol=0, atol=1e-12)


def test_one_shot_stack_selection_from_halt_layer():
    w = WORKLOADS[0].scaled(S=64, layers=3, halt_layer=1)
    get = lambda l: layer_inputs(w, 1, l)
    res = oracle.run_one_shot(get, 3, 1, k=20)
    x = get(1)
    s = np.sqrt(((oracle.causal_gqa_attention(x["Q"], x["K"], x["V"]) @ x["Wo"].astype(np.float64)) ** 2).sum(1))
    np.testing.assert_array_equal(res["idx"], brute_topk(s, 20))
    assert res["U"][2].shape == (20, w.hidden)


def test_decode_full_cache_is_dense_tail():
    """Keeping every token, decode rows equal the last rows of causal attention
    over the prefill followed by the new tokens."""
    w = WORKLOADS[0].scaled(S=40, Hq=4, Hkv=2, D=16, hidden=32)
    x = layer_inputs(w, 5, 0)
    y = layer_inputs(w.scaled(S=3), 6, 0)
    full = {n: np.concatenate([x[n], y[n]]) for n in ("Q", "K", "V")}
    dense = oracle.causal_gqa_attention(full["Q"], full["K"], full["V"])
    for mode in ("active", "all"):
        got = oracle.decode_step(y["Q"], y["K"], y["V"], x["K"], x["V"], np.arange(40), mode)
        np.testing.assert_allclose(got, dense[40:], rtol=0, atol=1e-12)


def test_decode_pruned_cache_brute_force():
    w = WORKLOADS[0].scaled(S=24, Hq=2, Hkv=1, D=8, hidden=16)
    x = layer_inputs(w, 7, 0)
    y = layer_inputs(w.scaled(S=2), 8, 0)
    idx = np.array([0, 3, 4, 9, 15, 23])
    got = oracle.decode_step(y["Q"], y["K"], y["V"], x["K"], x["V"], idx, "active")
    Kc = np.concatenate([x["K"][idx], y["K"]]).astype(np.float64)
    Vc = np.concatenate([x["V"][idx], y["V"]]).astype(np.float64)
    for i in range(2):
        visible = len(idx) + i + 1  # the cache plus the new tokens up to this one
        for h in range(2):
            sc = np.array([y["Q"][i, h].astype(np.float64) @ Kc[j, 0] for j in range(visible)]) / math.sqrt(8)
            p = np.exp(sc - sc.max())
            p /= p.sum()
            ref = sum(p[j] * Vc[j, 0] for j in range(visible))
            np.testing.assert_allclose(got[i, h * 8:(h + 1) * 8], ref, rtol=0, atol=1e-12)


def test_multi_shot_single_decision_is_one_shot():
    w = WORKLOADS[0].scaled(S=40, layers=3, halt_layer=1)
    get = lambda l: layer_inputs(w, 2, l)
    a = oracle.run_multi_shot(get, 3, [(1, 15)])
    b = oracle.run_one_shot(get, 3, 1, k=15)
    np.testing.assert_array_equal(a["idx"][0], b["idx"])
    np.testing.assert_allclose(a["U"][2], b["U"][2], rtol=0, atol=0)


def test_multi_shot_second_decision_brute_force():
    """The second decision, recomputed with explicit softmax attention over the
    first decision's rows (keys pruned to them), picks the top scores by the
    pairwise-rank rule."""
    w = WORKLOADS[0].scaled(S=48, Hq=2, Hkv=1, D=8, hidden=16, layers=4, halt_layer=0)
    get = lambda l: layer_inputs(w, 3, l)
    res = oracle.run_multi_shot(get, 4, [(0, 30), (2, 12)])
    idx1, idx2 = res["idx"]
    assert idx1.shape == (30,) and idx2.shape == (12,)
    assert set(idx2) <= set(idx1) and np.all(np.diff(idx2) > 0)
    x = get(2)
    Q, K, V = (x[n].astype(np.float64) for n in ("Q", "K", "V"))
    D = Q.shape[-1]
    rows = []
    for i, p in enumerate(idx1):
        heads = []
        for h in range(2):
            keys = idx1[idx1 <= p]
            sc = np.array([Q[p, h] @ K[j, 0] for j in keys]) / math.sqrt(D)
            pr = np.exp(sc - sc.max())
            pr /= pr.sum()
            heads.append(sum(pr[t] * V[j, 0] for t, j in enumerate(keys)))
        rows.append(np.concatenate(heads))
    U = np.array(rows) @ x["Wo"].astype(np.float64)
    s2 = np.sqrt((U * U).sum(1))
    np.testing.assert_array_equal(idx2, idx1[brute_topk(s2, 12)])
    # layer 3 runs on idx2 only
    assert res["U"][3].shape == (12, w.hidden)


def test_multi_shot_keep_all_is_dense():
    w = WORKLOADS[0].scaled(S=32, layers=4, halt_layer=0)
    get = lambda l: layer_inputs(w, 4, l)
    res = oracle.run_multi_shot(get, 4, [(0, 32), (2, 32)])
    x = get(3)
    _, U, _ = oracle.attention_layer(x["Q"], x["K"], x["V"], x["Wo"])
    np.testing.assert_allclose(res["U"][3], U, rtol=0, atol=1e-12)
    with pytest.raises(ValueError):
        oracle.run_multi_shot(get, 4, [(2, 10), (1, 5)])
    with pytest.raises(ValueError):
        oracle.run_multi_shot(get, 4, [(0, 10), (2, 20)])


def test_threshold_stack_min_tau_never_halts():
    w = WORKLOADS[3].scaled(S=32, Hq=4, Hkv=2, D=8, hidden=32, layers=4, dtype="f32")
    get = lambda l: layer_inputs(w, 0, l)
    res = oracle.run_threshold(get, 4, 32, tau_rank=1, patience=2)
    for p in res["pos"]:
        np.testing.assert_array_equal(p, np.arange(32))


def test_threshold_stack_halts_are_permanent_and_counted():
    w = WORKLOADS[3].scaled(S=48, Hq=4, Hkv=2, D=8, hidden=32, layers=5, dtype="f32")
    get = lambda l: layer_inputs(w, 2, l)
    res = oracle.run_threshold(get, 5, 48, tau_rank=oracle.percentile_rank(48, w.tau_pct), patience=2)
    for a, b in zip(res["pos"][:-1], res["pos"][1:]):
        assert set(b.tolist()) <= set(a.tolist())
    assert res["pos"][1].shape[0] == 48          # nobody halts before two layers have counted
    halted = set(range(48)) - set(res["final_pos"].tolist())
    assert all(res["counters"][p] == 2 for p in halted)


def test_threshold_stack_hand_worked_trajectory(golden_dir):
    """A whole selective-halting stack against a trajectory worked by hand
    (tests/golden/threshold_stack.json): with Q = 0 every query averages the
    values it can see, so each layer's scores are prefix means of V; K is
    random and must not matter."""
    g = json.load(open(os.path.join(golden_dir, "threshold_stack.json")))
    S = g["S"]
    rng = np.random.default_rng(5)

    def get(l):
        return {"Q": np.zeros((S, 1, 1)), "K": rng.standard_normal((S, 1, 1)),
                "V": np.asarray(g["V"][l], dtype=np.float64).reshape(S, 1, 1), "Wo": np.array([[g["Wo"]]])}

    L_ = len(g["V"])
    res = oracle.run_threshold(get, L_, S, tau_rank=g["tau_rank"], patience=g["patience"])
    assert res["tau"] == g["tau"]
    for l in range(L_):
        np.testing.assert_array_equal(res["pos"][l], g["pos"][l])
        np.testing.assert_allclose(res["score"][l], g["score"][l], rtol=0, atol=1e-12)
    np.testing.assert_array_equal(res["counters"], g["counters"])
    np.testing.assert_array_equal(res["final_pos"], g["final_pos"])


# ---------------------------------------------------------------------------
# generator sanity (data, not arithmetic)
# ---------------------------------------------------------------------------

def test_generator_deterministic_and_bf16_exact():
    w = WORKLOADS[1].scaled(S=64)
    a = layer_inputs(w, 0, 3)
    b = layer_inputs(w, 0, 3)
    for key in a:
        assert np.array_equal(a[key], b[key])
        assert np.array_equal(round_bf16(a[key]), a[key])
    assert a["Q"].shape == (64, 28, 128) and a["K"].shape == (64, 4, 128)
    assert a["Wo"].shape == (28 * 128, 3584)
    c = layer_inputs(w, 1, 3)
    assert not np.array_equal(a["Q"], c["Q"])
