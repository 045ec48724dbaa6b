#!/usr/bin/env python3
"""Benchmark of the DASH prefill hot path on one MI355X.

One step = one pass of the whole path over one synthetic sequence.  Default
workload (Qwen2.5-7B shapes, S=8192, bf16): the halting layer at full length
(causal GQA attention + W_o GEMM with the fused Δattn score), top-k selection
(keep 0.5), compaction of the next layer's K/V at the kept positions, and the
post-halt layer on the kept rows (attention reading its queries through the
kept indices + W_o, kv active).  `--config`
selects the other workloads: 0 = S=512 fp32; 2 = S=32768, 28 layers, halt at
layer 11; 3 = S=65536 Llama-3.1-8B shapes, 32 layers, threshold halting with
full K/V; 4 = S=131072, 28 layers, clustered salience, keep 0.3.

Prints one JSON line: prefill tokens/s of the step, the dense (no halting)
stack on the same kernels, a roofline entry for the dominant kernel (the
attention kernel, from HIP events the library records on its launch stream),
per-kernel timings, and the CPU oracle timed on this host as a reported
baseline.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "prefill tokens/s (halt + post-halt layers) vs dense; attn MFMA util; select GB/s"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3   # MI355X fp32 vector
PEAK_HBM_GBPS = 8000.0     # MI355X HBM3E
ATTN_SRC = os.path.join(ROOT, "attention_delta_token_amd", "csrc", "attn_fwd.hip")
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "attn_fwd_qwen_s8192_traffic.md")


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # ~30 steps (~30 ms at S=8192) bring the GPU to steady clocks; with 3 the
    # first timed steps run about 6% slow
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--config", type=int, default=1, choices=[0, 1, 2, 3, 4])
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--profile-only", action="store_true",
                    help="warmup + timed + traced steps only (for rocprofv3); no dense stack, no CPU leg")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one 512 MiB device-to-device copy (reference for HBM byte counters)")
    return ap.parse_args()


def attn_flops(D, Hq, n):
    """Algorithmic flops of causal attention over n rows: 4*D*Hq per (query, visible key) pair."""
    return 4.0 * D * Hq * n * (n + 1) / 2.0


def source_digest(path):
    """Digest of a kernel source's code: comments, blank lines and trailing
    spaces removed, so it changes with the kernel but not with its comments."""
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = [re.sub(r"//.*$", "", l).rstrip() for l in text.split("\n")]
    code = "\n".join(l for l in lines if l.strip())
    return hashlib.sha256(code.encode()).hexdigest()[:16]


def read_traffic(digest):
    """HBM bytes per attention launch from the committed counter summary, if it
    was taken on the current kernel source; else None."""
    try:
        text = open(TRAFFIC_PROFILE).read()
    except OSError:
        return None
    m = re.search(r"```json\n(.*?)\n```", text, re.S)
    if not m:
        return None
    data = json.loads(m.group(1))
    if data.get("attn_fwd_code_sha256_16") != digest:
        return None
    return data


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU (the path is built and measured on one device); --gpus must be 1",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)

    import torch
    import attention_delta_token_amd as dash
    from attention_delta_token_amd.stack import DenseStack, LayerTensors, OneShotStack, ThresholdStack
    from workload import WORKLOADS, layer_inputs

    dash.load()
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    w = WORKLOADS[args.config]
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32

    # Inputs: generated on the host layer by layer, uploaded, kept resident in HBM.
    keep_host = not args.no_cpu_baseline and not args.profile_only
    layers, host_keep = [], {}
    for l in range(w.layers):
        h = layer_inputs(w, args.seed, l)
        layers.append(LayerTensors(*(torch.from_numpy(h[n]).to(dev, tdt) for n in ("Q", "K", "V")),
                                   torch.from_numpy(np.ascontiguousarray(h["Wo"].T)).to(dev, tdt)))
        if keep_host and (l <= w.halt_layer + 1 or (w.mode == "threshold" and l <= 1)):
            host_keep[l] = h
        del h

    if w.mode == "threshold":
        step = ThresholdStack(layers, tau_rank=w.tau_rank, patience=w.patience)
    else:
        step = OneShotStack(layers, halt_layer=w.halt_layer, k=w.k)

    def timed(fn, steps):
        if torch.distributed.is_available() and torch.distributed.is_initialized():
            torch.distributed.barrier()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            fn()
        if torch.distributed.is_available() and torch.distributed.is_initialized():
            torch.distributed.barrier()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / steps

    if args.calibrate_copy:
        src = torch.empty(512 << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for _ in range(args.warmup):
        step.run()
    # The timed steps carry HIP events on the launch stream (torch's current
    # stream, which the binding passes to every call): one pair per step
    # (median and minimum step beside the mean) and the library's pair around
    # each attention launch, whose durations give the roofline entry.  Only the
    # attention launches are bracketed there, so the events cost the step as
    # little as possible; the per-kernel breakdown comes from the same steps
    # run again with every launch group bracketed.
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]

    def run_marked():
        i = run_marked.i
        if i == 0:
            ev[0].record()
        step.run()
        ev[i + 1].record()
        run_marked.i += 1
    run_marked.i = 0
    cap_attn = (w.layers + 1) * args.steps  # at most one attention launch per layer and step
    dash.trace_start(cap_attn)
    dash.trace_select(("attn_layer", "attn_active"))
    ms = timed(run_marked, args.steps)
    dash.trace_stop()
    # read right after the timed steps (context only); not under a profiler,
    # whose preloaded library would follow the rocm-smi child process
    clocks = gpu_clocks() if not args.profile_only else None
    attn_recs = dash.trace_read(cap_attn)
    per_step = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps))
    cap_all = (8 * w.layers + 8) * args.steps  # every launch group of every layer and step
    dash.trace_start(cap_all)
    ms_all_traced = timed(step.run, args.steps)
    dash.trace_stop()
    recs = dash.trace_read(cap_all)

    dense_ms = None
    if not args.no_dense and not args.profile_only:
        dense = DenseStack(layers)
        for _ in range(max(1, args.warmup)):
            dense.run()
        dense_ms = timed(dense.run, args.steps)

    # Gather-once step (one-shot policy): the kept rows' hidden states are
    # gathered once at the halting layer ([S, hidden] stand-in) and the
    # post-halt layers run on inputs compacted beforehand, as a model's own
    # projections would produce them; the main step above instead gathers each
    # post-halt layer's synthetic Q, K and V inside the step.
    gather_once_ms = None
    if w.mode != "threshold" and not args.profile_only and not args.no_dense:
        step.prepare_gather_once()
        for _ in range(args.warmup):
            step.run_gather_once()
        gather_once_ms = timed(step.run_gather_once, args.steps)

    S, Hq, Hkv, D, hid = w.S, w.Hq, w.Hkv, w.D, w.hidden
    by = {}
    for op, t in recs:
        by.setdefault(op, []).append(t)

    def avg(op):
        v = by.get(op, [])
        return (sum(v) / len(v)) if v else None

    # Algorithmic work per launch.
    f_full = attn_flops(D, Hq, S)
    proj_full = 2.0 * S * (Hq * D) * hid
    if w.mode == "threshold":
        # post-halt launches: queries = active set before each layer, keys = all positions <= query
        pos_trace = active_sets(step, layers)
        f_post_list = [4.0 * D * Hq * float(np.sum(p.astype(np.float64) + 1.0)) for p in pos_trace]
        f_post_layers = f_post_list
        proj_post_list = [2.0 * p.shape[0] * (Hq * D) * hid for p in pos_trace]
        n_full, k_rows = 1, [p.shape[0] for p in pos_trace]
    else:
        n_full = w.halt_layer + 1
        n_post = w.layers - n_full
        f_post_layers = [attn_flops(D, Hq, w.k)] * n_post
        proj_post_list = [2.0 * w.k * (Hq * D) * hid] * n_post
        k_rows = [w.k] * n_post
    # attention: the launches of the timed steps themselves
    by_attn = {}
    for op, t in attn_recs:
        by_attn.setdefault(op, []).append(t)
    t_full, t_post = by_attn.get("attn_layer", []), by_attn.get("attn_active", [])
    steps_traced = args.steps
    attn_flops_total = steps_traced * (n_full * f_full + sum(f_post_layers))
    attn_ms_total = sum(t_full) + sum(t_post)
    attn_launches = len(t_full) + len(t_post)
    attn_tflops = attn_flops_total / (attn_ms_total * 1e-3) / 1e12
    t_pl, t_pa = by.get("proj_layer", []), by.get("proj_active", [])
    proj_flops_total = steps_traced * (n_full * proj_full + sum(proj_post_list))
    proj_tflops = proj_flops_total / ((sum(t_pl) + sum(t_pa)) * 1e-3) / 1e12 if (t_pl or t_pa) else None
    esz = 2 if w.dtype == "bf16" else 4
    # select: 4 B per score read + 4 B per kept index (top-k); compaction: 2*row bytes + 4 B index per kept row.
    # The post-halt attention reads its queries through the kept indices, so only kv_mode active compacts
    # (K and V, in one launch); threshold mode (kv all) compacts nothing.
    if w.mode == "threshold":
        # order statistic: 4 B per layer-0 score; threshold step per active row: score 4 B + position 4 B
        # + counter read/write 2 B + surviving position 4 B
        sel_bytes_step = 4.0 * S + sum(14.0 * k for k in [S] + k_rows)
        n_sel_step = 2 + len(k_rows)
        cmp_bytes_step, n_cmp_step = 0.0, 0
    else:
        sel_bytes_step = 4.0 * S + 4.0 * w.k
        n_sel_step = 1
        if w.kv_mode == "active":
            cmp_bytes_step = sum(k * (2 * esz * 2 * Hkv * D + 4) for k in k_rows)
            n_cmp_step = len(k_rows)
        else:
            cmp_bytes_step, n_cmp_step = 0.0, 0
    t_sel, t_cmp = by.get("select", []), by.get("compact", [])
    sel_gbps = (steps_traced * sel_bytes_step) / (sum(t_sel) * 1e-3) / 1e9 if t_sel else None
    cmp_gbps = (steps_traced * cmp_bytes_step) / (sum(t_cmp) * 1e-3) / 1e9 if t_cmp else None

    dense_flops = w.layers * (f_full + proj_full)
    dash_flops = n_full * (f_full + proj_full) + sum(f_post_layers) + sum(proj_post_list)

    bf16 = w.dtype == "bf16"
    peak = PEAK_BF16_TFLOPS if bf16 else PEAK_FP32_TFLOPS
    digest = source_digest(ATTN_SRC)
    traffic = None
    tr = read_traffic(digest) if (args.config == 1) else None
    if tr is not None:
        traffic = tr["bytes_per_launch_avg"]

    out = {
        "metric": METRIC,
        "value": S / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) Q/K/V, lognormal V row scales, N(0,1/hidden) W_o; no trained weights)",
        "config": {"workload": describe(w), "global_batch": 1, "seq_len": S, "parallelism": "single GPU"},
        "roofline": {"bound": "mfma" if bf16 else "alu",
                     "kernel": f"attn_fwd_{'bf16' if bf16 else 'f32'}_kernel<{D}>",
                     "achieved": attn_tflops, "peak": peak, "unit": "TFLOP/s",
                     "frac": attn_tflops / peak, "traffic": traffic,
                     "launches": attn_launches, "avg_launch_ms": attn_ms_total / max(1, attn_launches),
                     "flops_per_launch_avg": attn_flops_total / max(1, attn_launches),
                     "attn_src_sha256_16": digest},
        "dense_ms_per_step": dense_ms,
        "dense_tokens_per_s": (S / (dense_ms * 1e-3)) if dense_ms else None,
        "speedup_vs_dense": (dense_ms / ms) if dense_ms else None,
        "ideal_speedup_flops": dense_flops / dash_flops,
        "gather_once": ({"ms_per_step": gather_once_ms, "tokens_per_s": S / (gather_once_ms * 1e-3),
                         "speedup_vs_dense": (dense_ms / gather_once_ms) if dense_ms else None,
                         "what": "one gather of an [S, hidden] bf16 hidden-state stand-in at the halting layer; "
                                 "post-halt layers on inputs compacted beforehand"}
                        if gather_once_ms else None),
        "all_traced_ms_per_step": ms_all_traced,
        "clocks_after_timed_steps": clocks,
        "step_ms_median": per_step[len(per_step) // 2], "step_ms_min": per_step[0],
        "kernels": {
            "attn_full_ms": (sum(t_full) / len(t_full)) if t_full else None,
            "attn_post_ms": (sum(t_post) / len(t_post)) if t_post else None,
            "attn_full_tflops": (f_full / (sum(t_full) / len(t_full) * 1e-3) / 1e12) if t_full else None,
            "attn_post_tflops": (steps_traced * sum(f_post_layers) / (sum(t_post) * 1e-3) / 1e12) if t_post else None,
            "proj_full_ms": avg("proj_layer"), "proj_post_ms": avg("proj_active"),
            "proj_tflops": proj_tflops, "proj_frac": (proj_tflops / peak) if proj_tflops else None,
            "select_ms": avg("select"), "select_calls_per_step": n_sel_step, "select_GBps": sel_gbps,
            "compact_ms": avg("compact"), "compact_calls_per_step": n_cmp_step, "compact_GBps": cmp_gbps,
            "compact_frac": (cmp_gbps / PEAK_HBM_GBPS) if cmp_gbps else None,
        },
        "active_rows_per_layer": k_rows if w.mode == "threshold" else None,
        "cpu_baseline": None,
    }

    if not args.profile_only:
        out["select_sweep"] = [select_sweep(dash, torch, dev, rows, n)
                               for rows, n in ((2048, 8192), (8192, 8192), (256, 65536))]
        out["score"] = score_measurements(dash, torch, dev, step, layers[0])
        if w.dtype == "bf16" and w.mode != "threshold":
            out["decode"] = decode_measurements(dash, torch, dev, w, layers[-1])

    if not args.no_cpu_baseline and not args.profile_only:
        out["cpu_baseline"] = cpu_baseline(w, host_keep, step, k_rows)

    print(json.dumps(out), flush=True)


def gpu_clocks():
    """Current shader and memory clocks as rocm-smi reports them (clocks are
    not pinned; recorded for context), or None when the tool is unavailable."""
    import subprocess
    try:
        r = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True, text=True, timeout=20)
        data = json.loads(r.stdout)
    except Exception:  # noqa: BLE001 - best effort only
        return None
    card = next(iter(data.values()), {}) if isinstance(data, dict) else {}
    return {k: v for k, v in card.items() if "sclk" in k.lower() or "mclk" in k.lower()} or None


def select_sweep(dash, torch, dev, rows=256, n=65536):
    """Top-k over a batch of independent score rows (one workgroup per row), the
    regime where selection is bandwidth-bound: 4 B read per score + 4 B written
    per kept index."""
    k = n // 2
    g = torch.Generator(device=dev).manual_seed(0)
    score = torch.rand(rows, n, device=dev, generator=g)
    idx = torch.empty(rows, k, dtype=torch.int32, device=dev)
    for _ in range(2):
        dash.dash_select(score, idx, mode=dash.DASH_SEL_TOPK, k=k, n_max=n, rows=rows)
    dash.trace_start(16)
    for _ in range(5):
        dash.dash_select(score, idx, mode=dash.DASH_SEL_TOPK, k=k, n_max=n, rows=rows)
    dash.trace_stop()
    t = [ms for op, ms in dash.trace_read(16) if op == "select"]
    ms = sum(t) / len(t)
    gbps = rows * (4.0 * n + 4.0 * k) / (ms * 1e-3) / 1e9
    return {"rows": rows, "n": n, "k": k, "ms": ms, "GBps": gbps, "frac": gbps / PEAK_HBM_GBPS}


def score_measurements(dash, torch, dev, step, layer):
    """The score two ways on the full-length layer: standalone (||U_t|| read back
    from a stored U: hidden * element size B read + 4 B written per row, HBM
    bound) and fused (the W_o GEMM with and without the sum of squares)."""
    U = step.U
    rows, hidden = U.shape
    score = torch.empty(rows, dtype=torch.float32, device=dev)
    for _ in range(3):
        dash.dash_score(U, score)
    dash.trace_start(64)
    for _ in range(20):
        dash.dash_score(U, score)
    dash.trace_stop()
    t = [ms for op, ms in dash.trace_read(64) if op == "score"]
    ms = sum(t) / len(t)
    gbps = rows * (hidden * U.element_size() + 4.0) / (ms * 1e-3) / 1e9
    # cold: a 1 GiB write before each call evicts U from L2 and the MALL
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    cold = []
    for i in range(5):
        flush.fill_(i)
        dash.trace_start(4)
        dash.dash_score(U, score)
        dash.trace_stop()
        cold.extend(t for op, t in dash.trace_read(4) if op == "score")
    del flush
    ms_cold = sum(cold) / len(cold)
    gbps_cold = rows * (hidden * U.element_size() + 4.0) / (ms_cold * 1e-3) / 1e9
    out = {"standalone_us": ms * 1e3, "standalone_GBps": gbps, "standalone_frac": gbps / PEAK_HBM_GBPS,
           "standalone_cold_us": ms_cold * 1e3, "standalone_cold_GBps": gbps_cold,
           "standalone_cold_frac": gbps_cold / PEAK_HBM_GBPS, "rows": rows, "hidden": hidden}
    # fused: the same layer's W_o GEMM with the score and without it
    ws = step.ws
    proj = {}
    for with_score in (True, False, True, False):
        dash.trace_start(64)
        for _ in range(10):
            dash.dash_attn_layer(layer.Q, layer.K, layer.V, layer.Wo, step.O, step.U,
                                 step.score if with_score else None, ws)
        dash.trace_stop()
        proj.setdefault(with_score, []).extend(ms for op, ms in dash.trace_read(64) if op == "proj_layer")
    with_ms = sum(proj[True]) / len(proj[True])
    without_ms = sum(proj[False]) / len(proj[False])
    out.update({"fused_proj_us": with_ms * 1e3, "plain_proj_us": without_ms * 1e3,
                "fused_overhead_us": (with_ms - without_ms) * 1e3})
    return out


def decode_measurements(dash, torch, dev, w, layer):
    """One decode token per sample against the cache a prefill leaves: the k kept
    rows (pruned) versus all S rows (dense), same kernels; the cache read (K and
    V of every cached row) is the algorithmic traffic.  A decode loop issues
    many small launches, so the calls are captured in a HIP graph (20 calls)
    and timed by replaying it on a busy GPU; each replay's output is checked
    against the eager call's."""
    res = {}
    Hkv, D, Hq = w.Hkv, w.D, w.Hq
    Qd = layer.Q[:1].reshape(1, 1, Hq, D).contiguous()
    for name, rows in (("pruned", w.k), ("dense", w.S)):  # cache rows, the new token's own included
        Kc = layer.K[:rows].reshape(1, rows, Hkv, D)
        Vc = layer.V[:rows].reshape(1, rows, Hkv, D)
        n_kv = torch.tensor([rows], dtype=torch.int32, device=dev)
        Od = torch.empty(1, 1, Hq * D, dtype=layer.Q.dtype, device=dev)
        ws = dash.workspace(dash.DASH_OP_DECODE, dash.make_shape(1, rows, Hq, Hkv, D, Hq * D, dash.DASH_BF16), 1,
                            device=dev)
        for _ in range(3):
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
        calls = 20
        with torch.cuda.graph(graph):
            for _ in range(calls):
                dash.dash_decode(Qd, Kc, Vc, n_kv, Od, ws=ws)
        for _ in range(3):
            Od.zero_()
            graph.replay()
            torch.cuda.synchronize()
            if not torch.equal(Od, ref):
                raise RuntimeError("decode graph replay differs from the eager call")
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 10
        e0.record()
        for _ in range(reps):
            graph.replay()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / (reps * calls)
        gbps = rows * Hkv * D * 2 * 2 / (ms * 1e-3) / 1e9
        res[name] = {"cache_rows": rows, "us": ms * 1e3, "cache_GBps": gbps}
        del graph
    res["speedup"] = res["dense"]["us"] / res["pruned"]["us"]
    res["timing"] = "HIP graph of 20 calls replayed 10 times (device time per call)"
    return res


def describe(w):
    s = (f"{w.name}: S={w.S}, Hq={w.Hq}, Hkv={w.Hkv}, D={w.D}, hidden={w.hidden}, {w.layers} layers, ")
    if w.mode == "threshold":
        return s + (f"threshold halting (tau = {w.tau_pct}th-percentile layer-0 score, patience {w.patience}), "
                    f"kv_mode={w.kv_mode}")
    return s + f"one-shot halt at layer {w.halt_layer}, top-k keep {w.keep} (k={w.k}), kv_mode={w.kv_mode}" + (
        ", clustered salience" if w.clustered else "")


def active_sets(step, layers):
    """Active query positions of each post-halt layer of the last threshold run (host copies)."""
    import torch  # noqa: F401
    st = step
    # Replay the run once, recording only the per-layer active sets.
    st.record, st.record_outputs = True, False
    st.trace = []
    st.run()
    st.record, st.record_outputs = False, True
    out = []
    for rec in st.trace[1:]:
        pos, n = rec[0], rec[1]
        out.append(pos[: int(n[0].item())].cpu().numpy())
    st.trace = []
    return out


def cpu_baseline(w, host_keep, step, k_rows):
    """The CPU oracle (float64 NumPy, as it stands) on the same seeded inputs."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    if w.S <= 8192:
        # whole steps (halting layer at full length + top-k + post-halt layer(s)), repeated until
        # about 10 s of CPU work has been timed (at most 4 repetitions)
        reps, t = 0, 0.0
        while reps < 4 and (reps == 0 or t < 10.0):
            t0 = time.perf_counter()
            x = host_keep[w.halt_layer]
            _, _, s = oracle.attention_layer(x["Q"], x["K"], x["V"], x["Wo"])
            idx = oracle.select_topk(s, w.k)
            for l in range(w.halt_layer + 1, w.layers):
                y = host_keep[l]
                oa = oracle.attn_active(y["Q"], y["K"], y["V"], idx, w.kv_mode)
                oracle.output_projection(oa, y["Wo"])
            t += time.perf_counter() - t0
            reps += 1
        per = t / reps
        est = per * (w.layers / (1 + (w.layers - w.halt_layer - 1))) if w.halt_layer > 0 else per
        sample = (f"{reps} whole step(s) of the same seeded workload (halt layer at full length + top-k + "
                  f"{w.layers - w.halt_layer - 1} post-halt layer), float64, {t:.1f} s in total")
        return {"value": w.S / est, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
                "sample": sample, "seconds": t}
    # Long sequences: time the oracle on a uniform sample of query rows of one full-length layer
    # and of one post-halt layer, and extrapolate to the stack.
    rng = np.random.default_rng(0)
    R = 64
    x = host_keep[w.halt_layer]
    rows = np.sort(rng.choice(w.S, R, replace=False))
    t0 = time.perf_counter()
    O = oracle.causal_gqa_attention(x["Q"][rows], x["K"], x["V"], q_pos=rows)
    oracle.delta_attn(oracle.output_projection(O, x["Wo"]))
    t_full_row = (time.perf_counter() - t0) / R
    y = host_keep[w.halt_layer + 1]
    if w.mode == "threshold":
        post_rows = np.sort(rng.choice(w.S, R, replace=False))
        t0 = time.perf_counter()
        O = oracle.causal_gqa_attention(y["Q"][post_rows], y["K"], y["V"], q_pos=post_rows)
        oracle.output_projection(O, y["Wo"])
        t_post_row = (time.perf_counter() - t0) / R
        n_full = 1
    else:
        k = w.k
        kidx = np.sort(rng.choice(w.S, k, replace=False))
        qsel = np.sort(rng.choice(k, R, replace=False))
        Ka, Va = y["K"][kidx], y["V"][kidx]
        t0 = time.perf_counter()
        O = oracle.causal_gqa_attention(y["Q"][kidx[qsel]], Ka, Va, q_pos=qsel)
        oracle.output_projection(O, y["Wo"])
        t_post_row = (time.perf_counter() - t0) / R
        n_full = w.halt_layer + 1
    est = n_full * w.S * t_full_row + sum(k_rows) * t_post_row
    return {"value": w.S / est, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": (f"{R} uniformly sampled query rows of one full-length layer and of one post-halt layer "
                       f"(float64), extrapolated to the {w.layers}-layer stack: {est:.0f} s"),
            "extrapolated": True}


if __name__ == "__main__":
    main()
