"""Seeded synthetic inputs for the DASH prefill path.

This module only draws random numbers and arranges them into arrays. It holds
none of the method's arithmetic (no attention, no norm, no selection), so the
CPU oracle and the HIP path can both consume exactly the same bits from it.

Every array is produced from a NumPy PCG64 stream keyed by
``SeedSequence([seed, cfg_id, layer, tensor_id])``; large tensors are drawn in
chunks of 2**22 elements, each chunk from its own spawned child seed, so the
values do not depend on the number of worker threads.

Values are drawn as float32.  For the bf16 workloads every value is rounded to
the nearest bf16 (ties to even) and returned as a float32 array whose values
are exactly representable in bf16: the oracle upcasts them to float64 and the
GPU side narrows them to bf16 without any further rounding.

Workload shapes (one sequence, B = 1):

* ``tiny``        S=512,    4 q-heads / 4 kv-heads, D=64,  hidden 256,  fp32
* ``qwen``        S=8192,  28 q-heads / 4 kv-heads, D=128, hidden 3584, bf16
* ``qwen28``      S=32768, Qwen2.5-7B shapes, 28 layers, one-shot halt at 11
* ``llama32``     S=65536, 32 q-heads / 8 kv-heads, D=128, hidden 4096, 32 layers,
                  threshold halting
* ``qwen28clust`` S=131072, Qwen2.5-7B shapes, 28 layers, clustered salience

Per layer: Q, K, V ~ N(0, 1); every token's V row (all kv-heads) is scaled by a
per-token factor f_t ~ lognormal(0, 1); W_o ~ N(0, 1/hidden) (the second
parameter read as the variance).  In the clustered workload 5 % of the tokens
lie in 256-token spans whose V rows are scaled by exactly 4, and all other rows
by lognormal(0, 0.5).
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace

import numpy as np

CHUNK = 1 << 22

T_Q, T_K, T_V, T_WO, T_VSCALE, T_SPANS, T_SCORE = 0, 1, 2, 3, 4, 5, 6


@dataclass(frozen=True)
class Workload:
    cfg_id: int
    name: str
    S: int
    Hq: int
    Hkv: int
    D: int
    hidden: int
    dtype: str            # "f32" or "bf16"
    layers: int
    mode: str             # "topk" (one-shot) or "threshold"
    halt_layer: int = 0   # one-shot: layers 0..halt_layer run full length
    keep: float = 0.5     # one-shot keep ratio (the kept count is the method's to derive)
    kv_mode: str = "active"
    tau_pct: int = 30            # threshold: tau = this percentile of the layer-0 scores
    patience: int = 2            # threshold: consecutive layers below tau before halting
    clustered: bool = False

    def scaled(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    0: Workload(0, "tiny", 512, 4, 4, 64, 256, "f32", 2, "topk", 0, 0.5, "active"),
    1: Workload(1, "qwen", 8192, 28, 4, 128, 3584, "bf16", 2, "topk", 0, 0.5, "active"),
    2: Workload(2, "qwen28", 32768, 28, 4, 128, 3584, "bf16", 28, "topk", 11, 0.5, "active"),
    3: Workload(3, "llama32", 65536, 32, 8, 128, 4096, "bf16", 32, "threshold", 0, 1.0, "all"),
    4: Workload(4, "qwen28clust", 131072, 28, 4, 128, 3584, "bf16", 28, "topk", 11, 0.3,
                "active", clustered=True),
}


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _stream(seed: int, cfg_id: int, layer: int, tensor_id: int) -> np.random.SeedSequence:
    return np.random.SeedSequence([seed, cfg_id, layer, tensor_id])


def normal_f32(ss: np.random.SeedSequence, n: int, std: float = 1.0, finish=None) -> np.ndarray:
    """n iid N(0, std^2) float32 values, chunked so the result is thread-count independent.

    finish(lo, hi, x), if given, is applied in place to each chunk x = out[lo:hi]
    right after it is drawn (on the worker thread that drew it); it must be
    elementwise, so the result does not depend on the chunking."""
    out = np.empty(n, dtype=np.float32)
    nchunks = max(1, (n + CHUNK - 1) // CHUNK)
    kids = ss.spawn(nchunks)

    def fill(c: int) -> None:
        lo, hi = c * CHUNK, min(n, (c + 1) * CHUNK)
        g = np.random.Generator(np.random.PCG64(kids[c]))
        g.standard_normal(hi - lo, dtype=np.float32, out=out[lo:hi])
        if std != 1.0:
            out[lo:hi] *= np.float32(std)
        if finish is not None:
            finish(lo, hi, out[lo:hi])

    if nchunks == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nchunks)))
    return out


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32 holding them.

    Finite inputs only (the generators never produce NaN or inf).
    """
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def _round_bf16_inplace(lo: int, hi: int, x: np.ndarray) -> None:
    x[:] = round_bf16(x)


def _finish(w: Workload):
    return _round_bf16_inplace if w.dtype == "bf16" else None


def span_slots(w: Workload, seed: int) -> np.ndarray:
    """Clustered workload: start positions of the salient 256-token spans (fixed per seed)."""
    nslots = w.S // 256
    nspans = int(round(0.05 * w.S / 256))
    nspans = max(1, min(nspans, nslots))
    g = np.random.Generator(np.random.PCG64(_stream(seed, w.cfg_id, 0, T_SPANS)))
    slots = np.sort(g.permutation(nslots)[:nspans])
    return slots * 256


def v_row_scale(w: Workload, seed: int, layer: int) -> np.ndarray:
    """Per-token multiplier applied to every kv-head of V[t] (float32, length S)."""
    g = np.random.Generator(np.random.PCG64(_stream(seed, w.cfg_id, layer, T_VSCALE)))
    if not w.clustered:
        return g.lognormal(0.0, 1.0, size=w.S).astype(np.float32)
    f = g.lognormal(0.0, 0.5, size=w.S).astype(np.float32)
    for s0 in span_slots(w, seed):
        f[s0:s0 + 256] = 4.0
    return f


def layer_inputs(w: Workload, seed: int, layer: int, parts=("Q", "K", "V", "Wo")) -> dict:
    """Q [S,Hq,D], K and V [S,Hkv,D], Wo [Hq*D, hidden] (U = O @ Wo), all float32 arrays.

    bf16 workloads: every value rounded to the nearest bf16 (V after its row
    scale is applied)."""
    out = {}
    S, Hq, Hkv, D, hid = w.S, w.Hq, w.Hkv, w.D, w.hidden
    fin = _finish(w)
    if "Q" in parts:
        out["Q"] = normal_f32(_stream(seed, w.cfg_id, layer, T_Q), S * Hq * D, finish=fin).reshape(S, Hq, D)
    if "K" in parts:
        out["K"] = normal_f32(_stream(seed, w.cfg_id, layer, T_K), S * Hkv * D, finish=fin).reshape(S, Hkv, D)
    if "V" in parts:
        scale = v_row_scale(w, seed, layer)
        row = Hkv * D

        def scale_then_round(lo: int, hi: int, x: np.ndarray) -> None:
            # element e of the flat [S, Hkv, D] array belongs to token e // (Hkv * D)
            tok = np.arange(lo, hi, dtype=np.int64) // row
            x *= scale[tok]
            if fin is not None:
                fin(lo, hi, x)

        out["V"] = normal_f32(_stream(seed, w.cfg_id, layer, T_V), S * Hkv * D,
                              finish=scale_then_round).reshape(S, Hkv, D)
    if "Wo" in parts:
        std = 1.0 / math.sqrt(hid)
        out["Wo"] = normal_f32(_stream(seed, w.cfg_id, layer, T_WO), Hq * D * hid, std,
                               finish=fin).reshape(Hq * D, hid)
    return out


# ---------------------------------------------------------------------------
# Score vectors that do not come from attention, for exercising selection on
# adversarial inputs (ties, signed zeros, permutations, special values).
# ---------------------------------------------------------------------------

def score_vector(kind: str, n: int, seed: int = 0) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(_stream(seed, 99, n, T_SCORE)))
    if kind == "normal":
        return np.abs(g.standard_normal(n, dtype=np.float32))
    if kind == "perm":
        return g.permutation(n).astype(np.float32)
    if kind == "equal":
        return np.full(n, 1.5, dtype=np.float32)
    if kind == "decreasing":
        return np.linspace(1.0, 0.0, n, dtype=np.float32) if n > 1 else np.ones(n, np.float32)
    if kind == "increasing":
        return np.linspace(0.0, 1.0, n, dtype=np.float32) if n > 1 else np.ones(n, np.float32)
    if kind == "fewvalues":
        return g.integers(0, 4, n).astype(np.float32)
    if kind == "signed":
        v = g.integers(-3, 4, n).astype(np.float32)
        v[g.random(n) < 0.2] = -0.0
        v[g.random(n) < 0.1] = 0.0
        return v
    if kind == "special":
        v = g.standard_normal(n, dtype=np.float32)
        r = g.random(n)
        v[r < 0.05] = np.inf
        v[(r >= 0.05) & (r < 0.10)] = -np.inf
        v[(r >= 0.10) & (r < 0.15)] = np.nan
        v[(r >= 0.15) & (r < 0.20)] = -0.0
        return v
    if kind == "denormal":
        return (g.integers(0, 50, n).astype(np.float32) * np.float32(1e-45))
    if kind == "bf16ties":
        return round_bf16(np.abs(g.standard_normal(n, dtype=np.float32)))
    raise ValueError(kind)


SCORE_KINDS = ("normal", "perm", "equal", "decreasing", "increasing", "fewvalues", "signed",
               "special", "denormal", "bf16ties")
