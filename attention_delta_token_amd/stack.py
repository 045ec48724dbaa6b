"""Drivers that chain the C-ABI calls into the DASH prefill stacks.

Only orchestration lives here (which call, on which buffers, in which
order); every step runs inside libdash.so.  Buffers are allocated once, up
front, so a step enqueues kernels only and never synchronises with the host.
Post-halt layers read their queries from the full-length Q through the kept
positions (dash_attn_active_gather); only a pruned KV cache (kv_mode active)
is compacted.

* One-shot policy (single-shot halting): layers 0..hl run at full length, the
  score of layer hl picks the k tokens to keep once, and layers hl+1..L-1 run
  on that active set — CSDN explainer "DASH：基于注意力增量的Transformer令牌压缩，
  实现长序列推理高效加速", §2.3 and §3.1.
* Threshold policy (selective halting): tau is an order statistic of the
  layer-0 scores; after every layer each active token's consecutive-below-tau
  counter is updated and tokens reaching `patience` stop being queries while
  keeping their K/V — forum summary "DASH：通过注意力动态监测实现长上下文高效预填充",
  sections 层间更新动态监测 and 选择性停止机制.
* Dense baseline: every layer at full length, no score/select/compact.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import _lib as L


@dataclass
class LayerTensors:
    """One layer's device inputs: Q [S,Hq,D], K and V [S,Hkv,D], Wo [hidden, Hq*D]."""
    Q: torch.Tensor
    K: torch.Tensor
    V: torch.Tensor
    Wo: torch.Tensor


def _shape_of(layer: LayerTensors):
    """(B, S, Hq, Hkv, D, hidden); Q is [S, Hq, D] (B = 1) or [B, S, Hq, D]."""
    if layer.Q.dim() == 4:
        B, S, Hq, D = layer.Q.shape
        return B, S, Hq, layer.K.shape[2], D, layer.Wo.shape[0]
    S, Hq, D = layer.Q.shape
    return 1, S, Hq, layer.K.shape[1], D, layer.Wo.shape[0]


class OneShotStack:
    """Layers 0..hl full length, top-k at hl (optionally forcing the first
    keep_first and last keep_last tokens in), layers hl+1..L-1 on the kept rows.
    Layers may hold one sample (Q [S, Hq, D]) or B samples of equal length
    (Q [B, S, Hq, D]); every sample keeps k = dash_keep_count(S, keep,
    keep_first, keep_last) tokens.  `status` receives each sample's count of
    NaN scores at the decision."""

    def __init__(self, layers: list[LayerTensors], halt_layer: int, keep: float, kv_mode: int = L.DASH_KV_ACTIVE,
                 keep_first: int = 0, keep_last: int = 0):
        self.layers = layers
        self.hl = halt_layer
        self.kv_mode = kv_mode
        self.keep_first, self.keep_last = keep_first, keep_last
        B, S, Hq, Hkv, D, hidden = _shape_of(layers[0])
        k = L.keep_count(S, keep, keep_first, keep_last)
        self.k = k  # total kept per sample, forced ends included
        dev, dt = layers[0].Q.device, layers[0].Q.dtype
        self.B, self.S, self.Hq, self.Hkv, self.D, self.hidden = B, S, Hq, Hkv, D, hidden
        lead = (B,) if layers[0].Q.dim() == 4 else ()
        kk = max(k, 1)
        self.O = torch.empty(*lead, S, Hq * D, device=dev, dtype=dt)
        self.U = torch.empty(*lead, S, hidden, device=dev, dtype=dt)
        self.score = torch.empty(*lead, S, device=dev, dtype=torch.float32)
        self.idx = torch.empty(*lead, kk, device=dev, dtype=torch.int32)
        self.Ka = torch.empty(*lead, kk, Hkv, D, device=dev, dtype=dt)
        self.Va = torch.empty(*lead, kk, Hkv, D, device=dev, dtype=dt)
        self.Oa = torch.empty(*lead, kk, Hq * D, device=dev, dtype=dt)
        self.Ua = torch.empty(*lead, kk, hidden, device=dev, dtype=dt)
        dtc = L.DASH_BF16 if dt == torch.bfloat16 else L.DASH_F32
        self.ws = L.workspace(L.DASH_OP_ATTN_LAYER, L.make_shape(B, S, Hq, Hkv, D, hidden, dtc), S, device=dev)
        self.status = L.select_status(B, device=dev, n_max=S)
        self.record_post = False  # keep a copy of every post-halt layer's Oa and Ua (tests)
        self.trace = []

    def full_layer(self, l: int, with_score: bool) -> None:
        x = self.layers[l]
        L.dash_attn_layer(x.Q, x.K, x.V, x.Wo, self.O, self.U, self.score if with_score else None, self.ws)

    def select(self) -> None:
        L.dash_select(self.score, self.idx, mode=L.DASH_SEL_TOPK, k=self.k, n_max=self.S, rows=self.B,
                      keep_first=self.keep_first, keep_last=self.keep_last, status=self.status)

    def post_layer(self, l: int) -> None:
        x = self.layers[l]
        k = self.k
        if k == 0:
            return
        batched = x.Q.dim() == 4
        # The queries are read from the full-length Q through the kept indices
        # inside the attention kernel; only kv_mode active compacts K and V.
        if self.kv_mode == L.DASH_KV_ACTIVE:
            pairs = [(x.K, self.Ka), (x.V, self.Va)]
            if batched:
                L.dash_compact_batch(self.idx, pairs)
            else:
                L.dash_compact_many(self.idx, pairs, n_max=k)
            L.dash_attn_active_gather(x.Q, self.idx, self.Ka, self.Va, L.DASH_KV_ACTIVE, self.Oa, n_max=k,
                                      Wo=x.Wo, Ua=self.Ua)
        else:
            L.dash_attn_active_gather(x.Q, self.idx, x.K, x.V, L.DASH_KV_ALL, self.Oa, q_pos=self.idx, n_max=k,
                                      Wo=x.Wo, Ua=self.Ua)

    def run(self) -> None:
        self.trace = []
        for l in range(len(self.layers)):
            if l <= self.hl:
                self.full_layer(l, with_score=(l == self.hl))
                if l == self.hl:
                    self.select()
            else:
                self.post_layer(l)
                if self.record_post:
                    self.trace.append((l, self.Oa.clone(), self.Ua.clone()))

    # -- gather once -------------------------------------------------------
    # A model gathers the hidden states of the kept tokens once at the halting
    # layer; every later layer's projections then produce compacted Q, K and V
    # by themselves.  The synthetic layers here hold full-length Q/K/V, so
    # run() gathers them per layer.  prepare_gather_once() takes the kept
    # indices of one run, gathers each post-halt layer's inputs once (outside
    # any timing), and run_gather_once() then does the step the way a model
    # would: full-length layers, selection, one gather of an [S, hidden]
    # hidden-state stand-in, post-halt layers on the already compacted inputs.

    def prepare_gather_once(self) -> None:
        if self.B != 1 or self.k == 0:
            raise ValueError("gather-once mode supports one sample with k > 0")
        self.run()
        torch.cuda.synchronize()
        dev, dt = self.O.device, self.O.dtype
        self.H = torch.zeros(self.S, self.hidden, device=dev, dtype=dt)  # hidden-state stand-in
        self.Ha = torch.empty(self.k, self.hidden, device=dev, dtype=dt)
        self.pre = {}
        for l in range(self.hl + 1, len(self.layers)):
            x = self.layers[l]
            Qa = torch.empty(self.k, self.Hq, self.D, device=dev, dtype=dt)
            if self.kv_mode == L.DASH_KV_ACTIVE:
                Ka = torch.empty(self.k, self.Hkv, self.D, device=dev, dtype=dt)
                Va = torch.empty(self.k, self.Hkv, self.D, device=dev, dtype=dt)
                L.dash_compact_many(self.idx, [(x.Q, Qa), (x.K, Ka), (x.V, Va)], n_max=self.k)
                self.pre[l] = (Qa, Ka, Va)
            else:
                L.dash_compact(self.idx, x.Q, Qa, n_max=self.k)
                self.pre[l] = (Qa, x.K, x.V)
        torch.cuda.synchronize()

    def run_gather_once(self) -> None:
        for l in range(len(self.layers)):
            if l <= self.hl:
                self.full_layer(l, with_score=(l == self.hl))
                if l == self.hl:
                    self.select()
                    L.dash_compact(self.idx, self.H, self.Ha, n_max=self.k)
            else:
                x, (Qa, Ka, Va) = self.layers[l], self.pre[l]
                if self.kv_mode == L.DASH_KV_ACTIVE:
                    L.dash_attn_active(Qa, Ka, Va, L.DASH_KV_ACTIVE, self.Oa, n_max=self.k, Wo=x.Wo, Ua=self.Ua)
                else:
                    L.dash_attn_active(Qa, Ka, Va, L.DASH_KV_ALL, self.Oa, q_pos=self.idx, n_max=self.k, Wo=x.Wo,
                                       Ua=self.Ua, S=self.S)


class RaggedOneShotStack:
    """One-shot halting for a packed batch of samples of different lengths:
    layers hold packed tensors (Q [T, Hq, D] ...) with the samples back to back
    (`lengths` on the host).  Every sample keeps its own
    k_b = dash_keep_count(len_b, keep, keep_first, keep_last) tokens (forced
    counts clamped to the sample); the kept rows stay packed (sample by
    sample) through the post-halt layers."""

    def __init__(self, layers: list[LayerTensors], lengths, halt_layer: int, keep: float,
                 kv_mode: int = L.DASH_KV_ACTIVE, keep_first: int = 0, keep_last: int = 0):
        self.layers = layers
        self.hl = halt_layer
        self.kv_mode = kv_mode
        self.keep_first, self.keep_last = keep_first, keep_last
        self.lengths = [int(n) for n in lengths]
        self.ks = [L.keep_count(n, keep, min(keep_first, n), min(keep_last, n - min(keep_first, n)))
                   for n in self.lengths]
        _, T, Hq, Hkv, D, hidden = _shape_of(layers[0])
        if T != sum(self.lengths):
            raise ValueError("packed rows do not match the sample lengths")
        dev, dt = layers[0].Q.device, layers[0].Q.dtype
        cu = [0]
        for n in self.lengths:
            cu.append(cu[-1] + n)
        cuk = [0]
        for k in self.ks:
            cuk.append(cuk[-1] + k)
        self.cu_seqlens = torch.tensor(cu, dtype=torch.int32, device=dev)
        self.cu_k = torch.tensor(cuk, dtype=torch.int32, device=dev)
        self.T, self.K = T, cuk[-1]
        self.max_len, self.max_k = max(self.lengths), max(max(self.ks), 1)
        kk = max(self.K, 1)
        self.O = torch.empty(T, Hq * D, device=dev, dtype=dt)
        self.U = torch.empty(T, hidden, device=dev, dtype=dt)
        self.score = torch.empty(T, device=dev, dtype=torch.float32)
        self.idx = torch.empty(kk, device=dev, dtype=torch.int32)
        self.Qa = torch.empty(kk, Hq, D, device=dev, dtype=dt)
        self.Ka = torch.empty(kk, Hkv, D, device=dev, dtype=dt)
        self.Va = torch.empty(kk, Hkv, D, device=dev, dtype=dt)
        self.Oa = torch.empty(kk, Hq * D, device=dev, dtype=dt)
        self.Ua = torch.empty(kk, hidden, device=dev, dtype=dt)
        dtc = L.DASH_BF16 if dt == torch.bfloat16 else L.DASH_F32
        self.ws = L.workspace(L.DASH_OP_ATTN_LAYER, L.make_shape(1, T, Hq, Hkv, D, hidden, dtc), T, device=dev)

    def full_layer(self, l: int, with_score: bool) -> None:
        x = self.layers[l]
        L.dash_attn_layer_varlen(x.Q, x.K, x.V, x.Wo, self.O, self.U, self.cu_seqlens, self.max_len,
                                 self.score if with_score else None, self.ws)

    def select(self) -> None:
        L.dash_select_ragged(self.score, self.idx, self.cu_seqlens, self.cu_k, self.max_len,
                             keep_first=self.keep_first, keep_last=self.keep_last)

    def post_layer(self, l: int) -> None:
        x = self.layers[l]
        if self.K == 0:
            return
        if self.kv_mode == L.DASH_KV_ACTIVE:
            L.dash_compact_many(self.idx, [(x.Q, self.Qa), (x.K, self.Ka), (x.V, self.Va)], n_max=self.K)
            L.dash_attn_active_varlen(self.Qa[:self.K], self.Ka[:self.K], self.Va[:self.K], L.DASH_KV_ACTIVE,
                                      self.Oa, self.cu_k, self.max_k, Wo=x.Wo, Ua=self.Ua)
        else:
            L.dash_compact(self.idx, x.Q, self.Qa, n_max=self.K)
            L.dash_attn_active_varlen(self.Qa[:self.K], x.K, x.V, L.DASH_KV_ALL, self.Oa, self.cu_k, self.max_k,
                                      q_pos=self.idx, cu_kv=self.cu_seqlens, Wo=x.Wo, Ua=self.Ua)

    def run(self) -> None:
        for l in range(len(self.layers)):
            if l <= self.hl:
                self.full_layer(l, with_score=(l == self.hl))
                if l == self.hl:
                    self.select()
            else:
                self.post_layer(l)


class MultiShotStack:
    """Halting decisions at several layers (one sample): schedule
    [(l_1, k_1), (l_2, k_2), ...] with increasing layers and non-increasing
    counts.  Layers 0..l_1 run at full length and layer l_1's scores keep k_1
    positions; each later decision layer scores its active rows and keeps the
    k_i best of them (top-k over the active rows, mapped to positions); the
    layers after a decision run on its set.  kv_mode active prunes the keys
    and values at every decision, kv_mode all keeps them."""

    def __init__(self, layers: list[LayerTensors], schedule, kv_mode: int = L.DASH_KV_ACTIVE):
        self.layers = layers
        self.schedule = list(schedule)
        self.kv_mode = kv_mode
        lays = [l for l, _ in self.schedule]
        if lays != sorted(set(lays)) or any(b[1] > a[1] for a, b in zip(self.schedule, self.schedule[1:])):
            raise ValueError("decision layers must increase and kept counts must not grow")
        B, S, Hq, Hkv, D, hidden = _shape_of(layers[0])
        if B != 1:
            raise ValueError("multi-shot stacks take one sample")
        dev, dt = layers[0].Q.device, layers[0].Q.dtype
        self.S = S
        k1 = max(self.schedule[0][1], 1)
        self.O = torch.empty(S, Hq * D, device=dev, dtype=dt)
        self.U = torch.empty(S, hidden, device=dev, dtype=dt)
        self.score = torch.empty(S, device=dev, dtype=torch.float32)
        self.pos = [torch.empty(max(k, 1), device=dev, dtype=torch.int32) for _, k in self.schedule]
        self.Ka = torch.empty(k1, Hkv, D, device=dev, dtype=dt)
        self.Va = torch.empty(k1, Hkv, D, device=dev, dtype=dt)
        self.Oa = torch.empty(k1, Hq * D, device=dev, dtype=dt)
        self.Ua = torch.empty(k1, hidden, device=dev, dtype=dt)
        dtc = L.DASH_BF16 if dt == torch.bfloat16 else L.DASH_F32
        self.ws = L.workspace(L.DASH_OP_ATTN_LAYER, L.make_shape(1, S, Hq, Hkv, D, hidden, dtc), S, device=dev)
        self.record = []  # (layer, position set, scores or None) per decision, device tensors
        self.keep_scores = False  # also copy each decision's scores (tests, measurement)

    def run(self) -> None:
        decisions = dict(self.schedule)
        self.record = []
        cur, n, d = None, self.S, 0
        for l, x in enumerate(self.layers):
            decide = l in decisions
            if cur is None:
                L.dash_attn_layer(x.Q, x.K, x.V, x.Wo, self.O, self.U, self.score if decide else None, self.ws)
            elif n > 0:
                if self.kv_mode == L.DASH_KV_ACTIVE:
                    L.dash_compact_many(cur, [(x.K, self.Ka), (x.V, self.Va)], n_max=n)
                    L.dash_attn_active_gather(x.Q, cur[:n], self.Ka[:n], self.Va[:n], L.DASH_KV_ACTIVE, self.Oa,
                                              n_max=n, Wo=x.Wo, Ua=self.Ua, score=self.score if decide else None,
                                              ws=self.ws)
                else:
                    L.dash_attn_active_gather(x.Q, cur[:n], x.K, x.V, L.DASH_KV_ALL, self.Oa, q_pos=cur, n_max=n,
                                              Wo=x.Wo, Ua=self.Ua, score=self.score if decide else None,
                                              ws=self.ws)
            if decide:
                k = decisions[l]
                nxt = self.pos[d]
                if k > 0:
                    L.dash_select(self.score, nxt, mode=L.DASH_SEL_TOPK, k=k, n_max=n, pos=cur)
                self.record.append((l, nxt, self.score[:n].clone() if self.keep_scores else None))
                cur, n, d = nxt, k, d + 1


class ThresholdStack:
    """Layer 0 full length fixes tau (the nearest-rank tau_pct-th percentile of
    its scores, dash_percentile_rank); every layer then updates the counters
    and runs on the surviving queries (read in place through their positions);
    keys and values stay full length (halted tokens keep their K/V).
    `status` receives the NaN counts of the last selection call."""

    def __init__(self, layers: list[LayerTensors], tau_pct: int, patience: int = 2, record: bool = False,
                 record_outputs: bool = True):
        self.layers = layers
        self.patience = patience
        _, S, Hq, Hkv, D, hidden = _shape_of(layers[0])
        self.rank = L.percentile_rank(S, tau_pct)
        dev, dt = layers[0].Q.device, layers[0].Q.dtype
        self.S = S
        self.O = torch.empty(S, Hq * D, device=dev, dtype=dt)
        self.U = torch.empty(S, hidden, device=dev, dtype=dt)
        self.score = torch.empty(S, device=dev, dtype=torch.float32)
        self.tau = torch.empty(4, device=dev, dtype=torch.float32)
        self.counters = torch.zeros(S, device=dev, dtype=torch.uint8)
        self.pos = [torch.empty(S, device=dev, dtype=torch.int32) for _ in range(2)]
        self.n = torch.zeros(2, 4, device=dev, dtype=torch.int32)
        self.Oa = torch.empty(S, Hq * D, device=dev, dtype=dt)
        dtc = L.DASH_BF16 if dt == torch.bfloat16 else L.DASH_F32
        self.ws = L.workspace(L.DASH_OP_ATTN_LAYER, L.make_shape(1, S, Hq, Hkv, D, hidden, dtc), S, device=dev)
        self.status = L.select_status(1, device=dev, n_max=S)
        self.record = record                  # keep per-layer host-visible copies (tests, measurement)
        self.record_outputs = record_outputs  # ... including scores and U, not only the active sets
        self.trace = []

    def run(self) -> None:
        S = self.S
        self.counters.zero_()
        x = self.layers[0]
        L.dash_attn_layer(x.Q, x.K, x.V, x.Wo, self.O, self.U, self.score, self.ws)
        L.dash_select(self.score, mode=L.DASH_SEL_ORDER_STAT, rank=self.rank, n_max=S, tau_out=self.tau)
        L.dash_select(self.score, self.pos[0], mode=L.DASH_SEL_THRESHOLD, tau=self.tau, patience=self.patience,
                      counters=self.counters, n_max=S, n_out=self.n[0], status=self.status)
        if self.record:
            self.trace.append((None, self.score.clone() if self.record_outputs else None))
        cur = 0
        for l in range(1, len(self.layers)):
            x = self.layers[l]
            pos, n = self.pos[cur], self.n[cur]
            L.dash_attn_active_gather(x.Q, pos, x.K, x.V, L.DASH_KV_ALL, self.Oa, q_pos=pos, n_dev=n, n_max=S,
                                      Wo=x.Wo, Ua=self.U, score=self.score, ws=self.ws)
            if self.record:
                if self.record_outputs:
                    self.trace.append((pos.clone(), n.clone(), self.score.clone(), self.U.clone()))
                else:
                    self.trace.append((pos.clone(), n.clone()))
            nxt = cur ^ 1
            L.dash_select(self.score, self.pos[nxt], mode=L.DASH_SEL_THRESHOLD, tau=self.tau,
                          patience=self.patience, counters=self.counters, pos=pos, n_dev=n, n_max=S,
                          n_out=self.n[nxt], status=self.status)
            cur = nxt
        self.final = cur


class DenseStack:
    """Every layer at full length (the comparison baseline)."""

    def __init__(self, layers: list[LayerTensors]):
        self.layers = layers
        B, S, Hq, Hkv, D, hidden = _shape_of(layers[0])
        dev, dt = layers[0].Q.device, layers[0].Q.dtype
        lead = (B,) if layers[0].Q.dim() == 4 else ()
        self.O = torch.empty(*lead, S, Hq * D, device=dev, dtype=dt)
        self.U = torch.empty(*lead, S, hidden, device=dev, dtype=dt)

    def run(self) -> None:
        for x in self.layers:
            L.dash_attn_layer(x.Q, x.K, x.V, x.Wo, self.O, self.U)
