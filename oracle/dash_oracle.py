"""Plain CPU oracle for the DASH prefill path (float64 NumPy).

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()`` and
the benchmark's ``cpu_baseline`` leg may import or call this module.  The
product path (the HIP library and its Python binding) never does, and this
module imports nothing from it: the two share no code.

Every function is the plain definition of one step, written for a reader to
check by eye; there is no blocking, fusion or reordering beyond processing
query rows in blocks to bound memory.  Sources (the web pages this method is
described on; cited by title and section):

* [P1] "DASH：基于注意力增量的Transformer令牌压缩，实现长序列推理高效加速"
  (CSDN blog explainer of Delta-Attention Single-shot Halting):
  §2.1 (what Δattn is), §2.3 (single-shot decision and start layer),
  §3.1 (algorithm walk-through), §3.2 (parameter table),
  §3.3 (PyTorch-style sketch of the prefill loop).
* [P2] "DASH：通过注意力动态监测实现长上下文高效预填充" (zingnex forum summary):
  sections "层间更新动态监测" (layer-wise update monitoring) and
  "选择性停止机制" (selective halting mechanism).
* [P3] "Stability Implies Redundancy: Delta Attention Selective Halting for
  Efficient Long-Context Prefilling" (abstract).

Readings taken where the pages are silent (each also listed in the design
notes): softmax scale 1/sqrt(D); q-head h reads kv-head h // (Hq/Hkv); U is the
attention output after the output projection and before the residual add, with
no bias; positions only mask (no rotary encoding); selection ties go to the
lower position; NaN scores rank below every number; ±0 compare equal; the
threshold uses a strict "<" and a consecutive-layer count that resets on any
layer at or above the threshold; halting is permanent.

Parity status: every function here is pinned by the CPU tests in
``tests/test_oracle_pins.py`` (brute force, closed forms, library routines and
the method's invariants).  None is "parity unpinned".
"""
from __future__ import annotations

import math

import numpy as np


# ---------------------------------------------------------------------------
# a1 / a5: causal grouped-query attention
# ---------------------------------------------------------------------------

def causal_gqa_attention(Q, K, V, q_pos=None, kv_pos=None, block_rows: int = 128) -> np.ndarray:
    """Causal GQA softmax attention, [P1] §2.1 (U is built from the attention
    module's output) and §3.1 (layers after the start layer attend over the
    active rows only).

    Q [n_q, Hq, D], K and V [n_kv, Hkv, D]; q_pos [n_q] and kv_pos [n_kv] are the
    original token positions (identity when None, kv_pos ascending).  For q-head
    h, kv-head j = h // (Hq // Hkv), and query row i:

        logits_r = (q_i · k_r) / sqrt(D)   for every key row r with kv_pos[r] <= q_pos[i]
        P_r      = exp(logits_r - max logits) / sum exp(...)
        O[i, h*D:(h+1)*D] = sum_r P_r v_r

    Returns O [n_q, Hq*D] in float64.  A query with no admissible key raises.
    """
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    n_q, Hq, D = Q.shape
    n_kv, Hkv, Dk = K.shape
    if Dk != D or V.shape != K.shape or Hq % Hkv != 0:
        raise ValueError("shape mismatch")
    g = Hq // Hkv
    q_pos = np.arange(n_q) if q_pos is None else np.asarray(q_pos, dtype=np.int64)
    kv_pos = np.arange(n_kv) if kv_pos is None else np.asarray(kv_pos, dtype=np.int64)
    if n_kv > 1 and np.any(np.diff(kv_pos) <= 0):
        raise ValueError("kv_pos must be strictly ascending")
    O = np.empty((n_q, Hq * D), dtype=np.float64)
    scale = 1.0 / math.sqrt(D)
    for b0 in range(0, n_q, block_rows):
        b1 = min(n_q, b0 + block_rows)
        qp = q_pos[b0:b1]
        # keys that any query of this block may see (kv_pos ascending)
        n_vis = int(np.searchsorted(kv_pos, qp.max(), side="right")) if b1 > b0 else 0
        mask = kv_pos[None, :n_vis] <= qp[:, None]
        if not np.all(mask.any(axis=1)):
            raise ValueError("a query has no admissible key")
        for h in range(Hq):
            j = h // g
            logits = (Q[b0:b1, h, :] @ K[:n_vis, j, :].T) * scale
            logits = np.where(mask, logits, -np.inf)
            m = logits.max(axis=1, keepdims=True)
            P = np.exp(logits - m)
            P /= P.sum(axis=1, keepdims=True)
            O[b0:b1, h * D:(h + 1) * D] = P @ V[:n_vis, j, :]
    return O


# ---------------------------------------------------------------------------
# a2: output projection and the Δattn score
# ---------------------------------------------------------------------------

def output_projection(O, Wo) -> np.ndarray:
    """U = O · W_o: the attention sublayer's update to the residual stream
    before the residual add, [P1] §2.1 (H' = H + U).  W_o is [Hq*D, hidden]."""
    return np.asarray(O, dtype=np.float64) @ np.asarray(Wo, dtype=np.float64)


def delta_attn(U) -> np.ndarray:
    """Δattn_t = ||U_t||_2, the Euclidean norm of token t's attention output
    row, [P1] §2.1 and §3.1 step 2; [P2] "层间更新动态监测" (the size of the
    layer's update to the token)."""
    U = np.asarray(U, dtype=np.float64)
    return np.sqrt(np.sum(U * U, axis=-1))


def attention_layer(Q, K, V, Wo, want_score: bool = True):
    """One full-length layer: O = attention, U = O·W_o, score = ||U_t||_2."""
    O = causal_gqa_attention(Q, K, V)
    U = output_projection(O, Wo)
    return O, U, (delta_attn(U) if want_score else None)


# ---------------------------------------------------------------------------
# a3: one-shot top-k selection
# ---------------------------------------------------------------------------

def topk_count(S: int, keep: float) -> int:
    """K = floor(keep * T), [P1] §3.1 step 3 (keep = 1 - pruning ratio ρ)."""
    return int(math.floor(keep * S))


def select_topk(score, k: int) -> np.ndarray:
    """The k positions with the largest score, returned in ascending position
    order, [P1] §2.3 and §3.1 step 3 (sort descending, keep the top K; the
    active index set is kept sorted, §3.3).  Ties go to the lower position;
    NaN ranks below every number; -0 and +0 are equal.

    Definition used: order all positions by the key (-score, position) and
    take the first k.  NumPy's stable argsort of -score is that order (it
    places NaN last and treats signed zeros as equal)."""
    s = np.asarray(score, dtype=np.float64)
    n = s.shape[0]
    if not 0 <= k <= n:
        raise ValueError("k out of range")
    order = np.argsort(-s, kind="stable")
    return np.sort(order[:k]).astype(np.int32)


def effective_keep_count(T: int, keep: float, keep_first: int, keep_last: int) -> int:
    """K_eff = f + l + floor(keep * (T - f - l)) with f = keep_first, l =
    keep_last and keep = 1 - ρ, [P1] §3.1 (forced retention of the first and
    last tokens, and the resulting kept count) and §3.3 (the sketch's total
    kept count).  Requires f + l <= T."""
    if keep_first < 0 or keep_last < 0 or keep_first + keep_last > T:
        raise ValueError("forced counts out of range")
    return keep_first + keep_last + int(math.floor(keep * (T - keep_first - keep_last)))


def select_topk_forced(score, k: int, keep_first: int, keep_last: int) -> np.ndarray:
    """Top-k with forced retention, [P1] §3.1 and §3.3: positions
    0..keep_first-1 and T-keep_last..T-1 are always kept, and the other
    k - keep_first - keep_last kept positions are the top ones among the
    middle positions keep_first..T-keep_last-1 (same order as select_topk:
    larger score first, ties to the lower position).  The result is the
    ascending union of the three sets (they are disjoint by construction).
    keep_last = 0 forces no tail token (the prose's meaning; the sketch's
    slice with 0 would mark every token)."""
    s = np.asarray(score, dtype=np.float64)
    n = s.shape[0]
    f, l = keep_first, keep_last
    if f < 0 or l < 0 or f + l > n or not f + l <= k <= n:
        raise ValueError("k or forced counts out of range")
    middle = s[f:n - l]
    dyn = select_topk(middle, k - f - l).astype(np.int64) + f
    head = np.arange(f)
    tail = np.arange(n - l, n)
    return np.concatenate([head, dyn, tail]).astype(np.int32)


def order_statistic(score, r: int) -> float:
    """τ = the r-th smallest score (1-based, nearest rank), with NaN ranking
    below every number and a zero returned as +0.  Used for the threshold of
    the selective-halting policy ([P2] "层间更新动态监测": a token halts when its
    update stays below a preset threshold)."""
    s = np.asarray(score, dtype=np.float64)
    n = s.shape[0]
    if not 1 <= r <= n:
        raise ValueError("rank out of range")
    nan = np.isnan(s)
    n_nan = int(nan.sum())
    if r <= n_nan:
        return float("nan")
    v = float(np.sort(s[~nan])[r - n_nan - 1])
    return 0.0 if v == 0.0 else v


def percentile_rank(S: int, pct: int) -> int:
    """Nearest-rank index of the pct-th percentile among S values,
    ceil(pct * S / 100), in integer arithmetic (0.3 * 10 is not exactly 3 in
    binary floating point)."""
    return max(1, -(-pct * S // 100))


# ---------------------------------------------------------------------------
# a3': threshold halting with consecutive-layer counters
# ---------------------------------------------------------------------------

def threshold_step(score_rows, pos, counters, tau: float, patience: int = 2):
    """One layer of selective halting, [P2] "层间更新动态监测" and "选择性停止机制":
    a token whose update stays below the threshold for `patience` consecutive
    layers halts; a halted token keeps its K/V but is no longer a query.

    score_rows[i] is the score of the active token at position pos[i] (pos
    ascending).  For each active token: c <- c + 1 if score < tau else 0; the
    token stays active iff c < patience.  Returns (new ascending active
    positions as int32, updated counters as uint8).  Counters of tokens that are
    not active are left unchanged."""
    score_rows = np.asarray(score_rows)
    pos = np.asarray(pos, dtype=np.int64)
    new_counters = np.array(counters, dtype=np.uint8, copy=True)
    keep = []
    for i in range(pos.shape[0]):
        p = int(pos[i])
        c = int(new_counters[p]) + 1 if score_rows[i] < tau else 0
        new_counters[p] = c
        if c < patience:
            keep.append(p)
    return np.asarray(keep, dtype=np.int32), new_counters


# ---------------------------------------------------------------------------
# a4: compaction
# ---------------------------------------------------------------------------

def compact(X, idx) -> np.ndarray:
    """Gather the active rows: Xa[r] = X[idx[r]], [P1] §3.1 step 4 (later
    layers take only the selected rows) and §3.3 (gather by active indices)."""
    X = np.asarray(X)
    return X[np.asarray(idx, dtype=np.int64)]


# ---------------------------------------------------------------------------
# a5: post-halt attention
# ---------------------------------------------------------------------------

def attn_active(Q, K, V, idx, kv_mode: str) -> np.ndarray:
    """Attention for the active tokens of a post-halt layer.

    Q, K, V are this layer's full-length [S, H, D] arrays and idx the ascending
    active positions.  Queries are Q[idx] at their original positions.
    * kv_mode "active": keys and values are K[idx], V[idx] — pruned tokens leave
      the KV cache, [P1] §3.1 step 4-5 and §5.1.
    * kv_mode "all": keys and values are all S rows — halted tokens stay in the
      KV cache but stop being queries, [P2] "选择性停止机制".
    Returns Oa [len(idx), Hq*D]."""
    idx = np.asarray(idx, dtype=np.int64)
    Qa = compact(Q, idx)
    if kv_mode == "active":
        return causal_gqa_attention(Qa, compact(K, idx), compact(V, idx), q_pos=idx, kv_pos=idx)
    if kv_mode == "all":
        return causal_gqa_attention(Qa, K, V, q_pos=idx, kv_pos=None)
    raise ValueError(kv_mode)


def decode_step(Q_new, K_new, V_new, K, V, idx, kv_mode: str) -> np.ndarray:
    """Attention of n_new decode tokens after a pruned prefill ([P1] §3.1 step 5
    and §5.1: the KV cache keeps only the active tokens, which also shortens
    decoding).  The prefill's cache is K[idx], V[idx] ("active", at positions
    idx) or all S rows ("all"); the new tokens' own K/V follow at positions
    S, S+1, ...; every key at a position at or before a query's is visible.
    Returns O [n_new, Hq*D]."""
    S = K.shape[0]
    n_new = Q_new.shape[0]
    idx = np.asarray(idx, dtype=np.int64)
    if kv_mode == "active":
        Kc, Vc, pos = compact(K, idx), compact(V, idx), idx
    elif kv_mode == "all":
        Kc, Vc, pos = np.asarray(K, np.float64), np.asarray(V, np.float64), np.arange(S)
    else:
        raise ValueError(kv_mode)
    new_pos = S + np.arange(n_new)
    Kc = np.concatenate([Kc, np.asarray(K_new, np.float64)])
    Vc = np.concatenate([Vc, np.asarray(V_new, np.float64)])
    return causal_gqa_attention(Q_new, Kc, Vc, q_pos=new_pos, kv_pos=np.concatenate([pos, new_pos]))


# ---------------------------------------------------------------------------
# Whole stacks (small sizes only): one-shot and threshold policies
# ---------------------------------------------------------------------------

def run_one_shot(get_layer, L: int, halt_layer: int, k: int, kv_mode: str = "active"):
    """One-shot policy, [P1] §2.3 and §3.1: layers 0..halt_layer run at full
    length, the score of layer halt_layer selects k tokens once, and layers
    halt_layer+1..L-1 run on that set only.

    get_layer(l) returns a dict with Q, K, V, Wo for layer l.  Returns a dict
    with the selected idx, the halt layer's score, and per-layer U (full-length
    for l <= halt_layer, active rows after)."""
    out = {"U": [], "O": []}
    idx = None
    for l in range(L):
        x = get_layer(l)
        if l <= halt_layer:
            O, U, s = attention_layer(x["Q"], x["K"], x["V"], x["Wo"], want_score=(l == halt_layer))
            if l == halt_layer:
                out["score"] = s
                idx = select_topk(s, k)
                out["idx"] = idx
        else:
            O = attn_active(x["Q"], x["K"], x["V"], idx, kv_mode)
            U = output_projection(O, x["Wo"])
        out["O"].append(O)
        out["U"].append(U)
    return out


def run_multi_shot(get_layer, L: int, schedule, kv_mode: str = "active"):
    """Halting decisions at several layers — the multi-round alternative to the
    single decision that [P1] §2.3 weighs against it, and the pruning at several
    key layers with growing ratios of [P1] §5.3.

    schedule = [(l_1, k_1), (l_2, k_2), ...] with l_1 < l_2 < ... and
    k_1 >= k_2 >= ...  Layers 0..l_1 run at full length and the score of layer
    l_1 keeps k_1 positions (select_topk).  Each later decision layer l_i is a
    post-halt layer: among its active rows it keeps the k_i with the largest
    score (same order as select_topk over those rows), and the layers after it
    run on that subset of positions.  With kv_mode "active" every decision also
    prunes the keys and values.

    Returns per-layer U and the position set chosen at each decision."""
    decisions = dict(schedule)
    layers = [l for l, _ in schedule]
    if layers != sorted(set(layers)) or any(b[1] > a[1] for a, b in zip(schedule, schedule[1:])):
        raise ValueError("decision layers must increase and kept counts must not grow")
    idx = None
    out = {"U": [], "idx": []}
    for l in range(L):
        x = get_layer(l)
        if idx is None:
            _, U, s = attention_layer(x["Q"], x["K"], x["V"], x["Wo"], want_score=(l in decisions))
        else:
            U = output_projection(attn_active(x["Q"], x["K"], x["V"], idx, kv_mode), x["Wo"])
            s = delta_attn(U)
        if l in decisions:
            keep = select_topk(s, decisions[l])
            idx = keep.astype(np.int32) if idx is None else idx[keep]
            out["idx"].append(idx)
        out["U"].append(U)
    return out


def run_threshold(get_layer, L: int, S: int, tau_rank: int, patience: int = 2, kv_mode: str = "all"):
    """Selective-halting policy, [P2] "层间更新动态监测" / "选择性停止机制": layer 0
    runs at full length and fixes τ as the tau_rank-th smallest layer-0 score;
    after every layer each active token's counter is updated and tokens whose
    counter reaches `patience` stop being queries from the next layer on.

    Returns per-layer active positions (the query set of each layer), scores,
    τ and the final counters."""
    counters = np.zeros(S, dtype=np.uint8)
    pos = np.arange(S, dtype=np.int32)
    out = {"pos": [], "score": [], "U": []}
    tau = None
    for l in range(L):
        x = get_layer(l)
        out["pos"].append(pos)
        if l == 0:
            _, U, s = attention_layer(x["Q"], x["K"], x["V"], x["Wo"])
            tau = order_statistic(s, tau_rank)
            out["tau"] = tau
        else:
            if pos.shape[0] == 0:
                U = np.zeros((0, x["Wo"].shape[1]))
                s = np.zeros(0)
            else:
                O = attn_active(x["Q"], x["K"], x["V"], pos, kv_mode)
                U = output_projection(O, x["Wo"])
                s = delta_attn(U)
        out["U"].append(U)
        out["score"].append(s)
        pos, counters = threshold_step(s, pos, counters, tau, patience)
    out["counters"] = counters
    out["final_pos"] = pos
    return out
