"""Runs the CPU oracle on many query rows at once, for the long-sequence parity
tests.  Test infrastructure only.

Attention heads are independent and every query row is computed on its own,
so the oracle's causal_gqa_attention is called on pieces: a block of query
rows (with their positions) for the q-heads of one kv-head against that
kv-head's keys and values.  The pieces run on a thread pool (NumPy releases
the interpreter lock inside its kernels) with the BLAS library held to one
thread per piece.  Nothing here computes attention itself: every number comes
from the oracle's own functions.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import oracle


def n_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def attention_rows(Q, K, V, q_rows, q_pos=None, kv_pos=None, rows_per_task: int = 256) -> np.ndarray:
    """Oracle attention output O [len(q_rows), Hq*D] (float64) for queries Q[q_rows]
    at positions q_pos (default: q_rows) against keys/values K, V at positions
    kv_pos (default: 0..n_kv-1)."""
    q_rows = np.asarray(q_rows, dtype=np.int64)
    q_pos = q_rows if q_pos is None else np.asarray(q_pos, dtype=np.int64)
    n, (_, Hq, D), Hkv = q_rows.shape[0], Q.shape, K.shape[1]
    g = Hq // Hkv
    out = np.empty((n, Hq * D), dtype=np.float64)
    if n == 0:
        return out
    kv_pos = np.arange(K.shape[0]) if kv_pos is None else np.asarray(kv_pos, dtype=np.int64)
    Kj = [np.ascontiguousarray(K[:, j:j + 1, :], dtype=np.float64) for j in range(Hkv)]
    Vj = [np.ascontiguousarray(V[:, j:j + 1, :], dtype=np.float64) for j in range(Hkv)]
    # queries in ascending position so each piece only touches the keys it can see
    order = np.argsort(q_pos, kind="stable")
    tasks = []
    for c0 in range(0, n, rows_per_task):
        sel = order[c0:c0 + rows_per_task]
        for j in range(Hkv):
            tasks.append((int(q_pos[sel].max()), sel, j))
    tasks.sort(key=lambda t: -t[0])  # heaviest first

    def run(t):
        _, sel, j = t
        vis = int(np.searchsorted(kv_pos, q_pos[sel].max(), side="right"))
        Qs = np.asarray(Q[q_rows[sel]][:, j * g:(j + 1) * g, :], dtype=np.float64)
        o = oracle.causal_gqa_attention(Qs, Kj[j][:vis], Vj[j][:vis], q_pos=q_pos[sel], kv_pos=kv_pos[:vis])
        out[sel, j * g * D:(j + 1) * g * D] = o

    try:
        from threadpoolctl import threadpool_limits
        limit = threadpool_limits(limits=1, user_api="blas")
    except Exception:  # pragma: no cover - threadpoolctl missing
        limit = None
    try:
        with ThreadPoolExecutor(n_threads()) as ex:
            list(ex.map(run, tasks))
    finally:
        if limit is not None:
            limit.restore_original_limits()
    return out


def layer_rows(x, q_rows, q_pos=None, kv_rows=None):
    """Oracle O, U = O·W_o and score = ||U_t|| for the given query rows of one
    layer x (a dict with Q, K, V, Wo).  kv_rows: the key/value rows kept (an
    ascending index list, kv_mode active); None keeps all rows."""
    if kv_rows is None:
        O = attention_rows(x["Q"], x["K"], x["V"], q_rows, q_pos)
    else:
        kv_rows = np.asarray(kv_rows, dtype=np.int64)
        O = attention_rows(x["Q"], x["K"][kv_rows], x["V"][kv_rows], q_rows, q_pos, kv_pos=kv_rows)
    U = oracle.output_projection(O, x["Wo"])
    return O, U, oracle.delta_attn(U)
