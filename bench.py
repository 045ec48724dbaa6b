#!/usr/bin/env python3
"""Benchmark of the DASH prefill hot path on one MI355X.

One step = one pass of the whole path over one synthetic sequence.  Default
workload (the largest one, Qwen2.5-7B shapes, bf16): S=131072 tokens, 28
layers, clustered salience; layers 0..11 at full length (causal GQA attention
+ W_o GEMM, with the fused Δattn score at layer 11), top-k selection (keep
0.3, k=39321), then layers 12..27 on the kept rows (K/V gathered at the kept
positions, attention reading its queries through the kept indices, W_o on the
kept rows).  `--config` selects the other workloads: 0 = S=512 fp32; 1 =
S=8192, halt layer + one post-halt layer; 2 = S=32768, 28 layers, halt at 11;
3 = S=65536 Llama-3.1-8B shapes, 32 layers, threshold halting with full K/V.

Prints one JSON line: prefill tokens/s of the step, the dense (no halting)
stack on the same kernels timed in alternation with the step, a roofline
entry for the dominant kernel (the attention kernel, from HIP events the
library records on its launch stream), per-kernel timings, and the CPU oracle
timed on this host as a reported baseline.
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


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=4, choices=[0, 1, 2, 3, 4])
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--profile-only", action="store_true",
                    help="warmup + timed + traced steps only (for rocprofv3); no dense stack, no CPU leg")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one 512 MiB device-to-device copy (reference for HBM byte counters)")
    ap.add_argument("--hbm-kernels", action="store_true",
                    help="only the HBM-bound kernels on synthetic inputs of the workload's shapes (batched "
                         "top-k sweep, standalone score, K/V gather), warm and cold; one JSON line")
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


def traffic_profile(w):
    return os.path.join(ROOT, "profiles", f"attn_fwd_{w.name}_s{w.S}_traffic.md")


def read_traffic(w, digest):
    """HBM bytes per attention launch from the committed counter summary of this
    workload, if it was taken on the current kernel source; else None."""
    try:
        text = open(traffic_profile(w)).read()
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
    if args.hbm_kernels:
        hbm_kernels(dash, torch, dev, w, args)
        return

    # Inputs: generated on the host layer by layer, narrowed to the element
    # type on the host (the values are exact in it), uploaded, kept resident.
    t_gen = time.perf_counter()
    keep_host = not args.no_cpu_baseline and not args.profile_only
    layers, host_keep = [], {}
    for l in range(w.layers):
        h = layer_inputs(w, args.seed, l)
        layers.append(LayerTensors(*(torch.from_numpy(h[n]).to(tdt).to(dev) for n in ("Q", "K", "V")),
                                   torch.from_numpy(np.ascontiguousarray(h["Wo"].T)).to(tdt).to(dev)))
        if keep_host and (l in (w.halt_layer, w.halt_layer + 1) or (w.mode == "threshold" and l <= 1)):
            host_keep[l] = h
        del h
    torch.cuda.synchronize()
    print(f"# {w.name}: {w.layers} layers generated and uploaded in {time.perf_counter() - t_gen:.1f} s",
          file=sys.stderr, flush=True)

    if w.mode == "threshold":
        step = ThresholdStack(layers, tau_pct=w.tau_pct, patience=w.patience)
    else:
        step = OneShotStack(layers, halt_layer=w.halt_layer, keep=w.keep)

    def timed(fn, steps, clocks=False):
        """Wall-clock ms per step over `steps` calls bracketed by synchronisations.
        clocks: a side thread reads rocm-smi 2 s into the region (context only;
        the timed thread never waits for it)."""
        import threading
        got = {}

        def sample():
            time.sleep(2.0)
            got["clocks"] = gpu_clocks()
            got["at_s"] = time.perf_counter() - t0
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        th = threading.Thread(target=sample, daemon=True) if clocks else None
        if th:
            th.start()
        for _ in range(steps):
            fn()
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        c = None
        if th:
            th.join()
            c = {"rocm_smi": got.get("clocks"), "read_at_s": got.get("at_s"), "timed_region_s": elapsed}
        return elapsed * 1e3 / steps, c

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
    # little as possible; the per-kernel breakdown comes from a few more steps
    # run with every launch group bracketed.
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
    # not under a profiler: its preloaded library would follow the rocm-smi child
    ms, clocks = timed(run_marked, args.steps, clocks=not args.profile_only)
    dash.trace_stop()
    attn_recs = dash.trace_read(cap_attn)
    per_step = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps))
    n_traced = max(1, min(args.steps, 3))
    cap_all = (8 * w.layers + 8) * n_traced  # every launch group of every layer and step
    dash.trace_start(cap_all)
    ms_all_traced, _ = timed(step.run, n_traced)
    dash.trace_stop()
    recs = dash.trace_read(cap_all)

    # Dense comparison: the dense stack (every layer at full length, same
    # kernels) and the DASH step in alternation, so both see the same clock
    # and thermal state; each step bracketed by events on the launch stream.
    cmp = None
    if not args.no_dense and not args.profile_only:
        dense = DenseStack(layers)
        dense.run()
        pairs = max(2, min(args.steps, 6))
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(4 * pairs)]
        torch.cuda.synchronize()
        for i in range(pairs):
            evs[4 * i].record()
            step.run()
            evs[4 * i + 1].record()
            evs[4 * i + 2].record()
            dense.run()
            evs[4 * i + 3].record()
        torch.cuda.synchronize()
        d_ms = [evs[4 * i].elapsed_time(evs[4 * i + 1]) for i in range(pairs)]
        n_ms = [evs[4 * i + 2].elapsed_time(evs[4 * i + 3]) for i in range(pairs)]
        cmp = {"pairs": pairs, "dash_ms": sum(d_ms) / pairs, "dense_ms": sum(n_ms) / pairs,
               "speedup": sum(n_ms) / sum(d_ms)}
        del dense

    # Gather-once step (one-shot policy): the kept rows' hidden states are
    # gathered once at the halting layer ([S, hidden] stand-in) and the
    # post-halt layers run on inputs compacted beforehand, as a model's own
    # projections would produce them; the main step above instead gathers each
    # post-halt layer's synthetic K and V inside the step.
    gather_once_ms = None
    if w.mode != "threshold" and not args.profile_only and not args.no_dense:
        step.prepare_gather_once()
        step.run_gather_once()
        gather_once_ms, _ = timed(step.run_gather_once, max(1, min(args.steps, 3)))
        step.pre, step.H, step.Ha = {}, None, None

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
        pos_trace = active_sets(step)
        f_post_layers = [4.0 * D * Hq * float(np.sum(p.astype(np.float64) + 1.0)) for p in pos_trace]
        proj_post_list = [2.0 * p.shape[0] * (Hq * D) * hid for p in pos_trace]
        n_full, k_rows = 1, [p.shape[0] for p in pos_trace]
    else:
        n_full = w.halt_layer + 1
        n_post = w.layers - n_full
        f_post_layers = [attn_flops(D, Hq, step.k)] * n_post
        proj_post_list = [2.0 * step.k * (Hq * D) * hid] * n_post
        k_rows = [step.k] * n_post
    # attention: the launches of the timed steps themselves
    by_attn = {}
    for op, t in attn_recs:
        by_attn.setdefault(op, []).append(t)
    t_full, t_post = by_attn.get("attn_layer", []), by_attn.get("attn_active", [])
    attn_flops_total = args.steps * (n_full * f_full + sum(f_post_layers))
    attn_ms_total = sum(t_full) + sum(t_post)
    attn_launches = len(t_full) + len(t_post)
    attn_tflops = attn_flops_total / (attn_ms_total * 1e-3) / 1e12
    t_pl, t_pa = by.get("proj_layer", []), by.get("proj_active", [])
    proj_flops_total = n_traced * (n_full * proj_full + sum(proj_post_list))
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
        sel_bytes_step = 4.0 * S + 4.0 * step.k
        n_sel_step = 1
        if w.kv_mode == "active":
            cmp_bytes_step = sum(k * (2 * esz * 2 * Hkv * D + 4) for k in k_rows)
            n_cmp_step = len(k_rows)
        else:
            cmp_bytes_step, n_cmp_step = 0.0, 0
    t_sel, t_cmp = by.get("select", []), by.get("compact", [])
    sel_gbps = (n_traced * sel_bytes_step) / (sum(t_sel) * 1e-3) / 1e9 if t_sel else None
    cmp_gbps = (n_traced * cmp_bytes_step) / (sum(t_cmp) * 1e-3) / 1e9 if t_cmp else None

    dense_flops = w.layers * (f_full + proj_full)
    dash_flops = n_full * (f_full + proj_full) + sum(f_post_layers) + sum(proj_post_list)

    bf16 = w.dtype == "bf16"
    peak = PEAK_BF16_TFLOPS if bf16 else PEAK_FP32_TFLOPS
    digest = source_digest(ATTN_SRC)
    tr = read_traffic(w, digest)
    traffic = tr["bytes_per_launch_avg"] if tr is not None else None

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
        "config": {"workload": describe(w, step), "global_batch": 1, "seq_len": S, "parallelism": "single GPU"},
        "roofline": {"bound": "mfma" if bf16 else "alu",
                     "kernel": f"attn_fwd_{'bf16_pp' if bf16 else 'f32'}_kernel<{D}>",
                     "achieved": attn_tflops, "peak": peak, "unit": "TFLOP/s",
                     "frac": attn_tflops / peak, "traffic": traffic,
                     "launches": attn_launches, "avg_launch_ms": attn_ms_total / max(1, attn_launches),
                     "flops_per_launch_avg": attn_flops_total / max(1, attn_launches),
                     "attn_src_sha256_16": digest},
        "dense_ms_per_step": cmp["dense_ms"] if cmp else None,
        "dense_tokens_per_s": (S / (cmp["dense_ms"] * 1e-3)) if cmp else None,
        "speedup_vs_dense": cmp["speedup"] if cmp else None,
        "dense_comparison": ({"how": f"{cmp['pairs']} DASH steps and {cmp['pairs']} dense steps in alternation, "
                                     "HIP events around each",
                              "dash_ms": cmp["dash_ms"], "dense_ms": cmp["dense_ms"]} if cmp else None),
        "ideal_speedup_flops": dense_flops / dash_flops,
        "gather_once": ({"ms_per_step": gather_once_ms, "tokens_per_s": S / (gather_once_ms * 1e-3),
                         "speedup_vs_dense": (cmp["dense_ms"] / gather_once_ms) if cmp else None,
                         "what": "one gather of an [S, hidden] bf16 hidden-state stand-in at the halting layer; "
                                 "post-halt layers on inputs compacted beforehand"}
                        if gather_once_ms else None),
        "all_traced_ms_per_step": ms_all_traced,
        "clocks_during_timed_steps": clocks,
        "step_ms_median": per_step[len(per_step) // 2], "step_ms_min": per_step[0],
        "kernels": {
            "attn_full_ms": (sum(t_full) / len(t_full)) if t_full else None,
            "attn_post_ms": (sum(t_post) / len(t_post)) if t_post else None,
            "attn_full_tflops": (f_full / (sum(t_full) / len(t_full) * 1e-3) / 1e12) if t_full else None,
            "attn_full_frac": (f_full / (sum(t_full) / len(t_full) * 1e-3) / 1e12 / peak) if t_full else None,
            "attn_post_tflops": (args.steps * sum(f_post_layers) / (sum(t_post) * 1e-3) / 1e12) if t_post else None,
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
        out["score"] = score_measurements(dash, torch, dev, step, layers[w.halt_layer if w.mode != "threshold" else 0])
        if w.dtype == "bf16" and w.mode != "threshold":
            out["decode"] = decode_measurements(dash, torch, dev, w, layers[-1], step.k)

    if not args.no_cpu_baseline and not args.profile_only:
        out["cpu_baseline"] = cpu_baseline(w, host_keep, step, k_rows)

    print(json.dumps(out), flush=True)


def gpu_clocks():
    """Current shader and memory clocks and the package power as rocm-smi
    reports them (clocks are not pinned; recorded for context), or None when
    the tool is unavailable."""
    import subprocess
    try:
        r = subprocess.run(["rocm-smi", "--showclocks", "--showpower", "--showmaxpower", "--json"], capture_output=True, text=True,
                           timeout=20)
        data = json.loads(r.stdout)
    except Exception:  # noqa: BLE001 - best effort only
        return None
    card = next(iter(data.values()), {}) if isinstance(data, dict) else {}
    keep = ("sclk", "mclk", "power")
    return {k: v for k, v in card.items() if any(x in k.lower() for x in keep)} or None


def select_sweep(dash, torch, dev, rows=256, n=65536):
    """Top-k over a batch of independent score rows, the regime where selection
    is bandwidth-bound: 4 B read per score + 4 B written per kept index."""
    k = n // 2
    g = torch.Generator(device=dev).manual_seed(0)
    score = torch.rand(rows, n, device=dev, generator=g)
    idx = torch.empty(rows, k, dtype=torch.int32, device=dev)
    for _ in range(2):
        dash.dash_select(score, idx, mode=dash.DASH_SEL_TOPK, k=k, n_max=n, rows=rows)
    # throughput: 10 calls back to back between one pair of events on the
    # stream the library launches on (torch's current stream)
    reps = 10
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(reps):
        dash.dash_select(score, idx, mode=dash.DASH_SEL_TOPK, k=k, n_max=n, rows=rows)
    ev1.record()
    ev1.synchronize()
    ms = ev0.elapsed_time(ev1) / reps
    # one call at a time (HIP events around each launch; includes the launch latency)
    dash.trace_start(16)
    for _ in range(5):
        dash.dash_select(score, idx, mode=dash.DASH_SEL_TOPK, k=k, n_max=n, rows=rows)
    dash.trace_stop()
    t = [m for op, m in dash.trace_read(16) if op == "select"]
    gbps = rows * (4.0 * n + 4.0 * k) / (ms * 1e-3) / 1e9
    return {"rows": rows, "n": n, "k": k, "ms": ms, "GBps": gbps, "frac": gbps / PEAK_HBM_GBPS,
            "ms_single_call": sum(t) / len(t), "timing": f"{reps} calls back to back, events around the batch"}


def timed_calls(torch, fn, reps, flush=None):
    """Mean ms per call: `reps` calls back to back between one pair of events
    (warm), or, with a flush buffer, each call alone after a write of the whole
    buffer (cold: the inputs are evicted from L2 and the MALL)."""
    fn()
    if flush is None:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        e1.synchronize()
        return e0.elapsed_time(e1) / reps
    t = 0.0
    for i in range(reps):
        flush.fill_(i & 0xff)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        e1.synchronize()
        t += e0.elapsed_time(e1)
    return t / reps


def hbm_kernels(dash, torch, dev, w, args):
    """The HBM-bound kernels alone, on synthetic inputs of the workload's
    shapes (values do not change their traffic): the batched top-k sweep, the
    standalone score over an [S, hidden] U, and the one-launch gather of the
    kept rows' K and V (k = the one-shot kept count), each warm and after a
    1 GiB write.  Algorithmic bytes: top-k 4 B per score + 4 B per kept index;
    score hidden * element size + 4 B per row; gather 2 * 2 * Hkv * D * element
    size + 4 B per kept row."""
    g = torch.Generator(device=dev).manual_seed(args.seed)
    esz = 2 if w.dtype == "bf16" else 4
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    out = {"workload": f"{w.name}: S={w.S}, Hq={w.Hq}, Hkv={w.Hkv}, D={w.D}, hidden={w.hidden}",
           "peak_GBps": PEAK_HBM_GBPS, "select_sweep": [], "timing": "warm: 10 calls back to back between one "
           "pair of events; cold: each call alone after a 1 GiB write"}
    for rows, n in ((2048, 8192), (8192, 8192), (256, 65536)):
        k = n // 2
        score = torch.rand(rows, n, device=dev, generator=g)
        idx = torch.empty(rows, k, dtype=torch.int32, device=dev)
        fn = lambda: dash.dash_select(score, idx, mode=dash.DASH_SEL_TOPK, k=k, n_max=n, rows=rows)
        nbytes = rows * (4.0 * n + 4.0 * k)
        warm, cold = timed_calls(torch, fn, 10), timed_calls(torch, fn, 5, flush)
        out["select_sweep"].append({"rows": rows, "n": n, "k": k, "bytes": nbytes, "ms": warm, "ms_cold": cold,
                                    "frac": nbytes / (warm * 1e-3) / 1e9 / PEAK_HBM_GBPS,
                                    "frac_cold": nbytes / (cold * 1e-3) / 1e9 / PEAK_HBM_GBPS})
        del score, idx
    U = torch.randn(w.S, w.hidden, device=dev, generator=g).to(tdt)
    sc = torch.empty(w.S, dtype=torch.float32, device=dev)
    fn = lambda: dash.dash_score(U, sc)
    nbytes = w.S * (w.hidden * esz + 4.0)
    warm, cold = timed_calls(torch, fn, 10), timed_calls(torch, fn, 5, flush)
    out["score"] = {"rows": w.S, "hidden": w.hidden, "bytes": nbytes, "ms": warm, "ms_cold": cold,
                    "frac": nbytes / (warm * 1e-3) / 1e9 / PEAK_HBM_GBPS,
                    "frac_cold": nbytes / (cold * 1e-3) / 1e9 / PEAK_HBM_GBPS}
    del U, sc
    k = dash.keep_count(w.S, w.keep)
    K = torch.randn(w.S, w.Hkv, w.D, device=dev, generator=g).to(tdt)
    V = torch.randn(w.S, w.Hkv, w.D, device=dev, generator=g).to(tdt)
    kept = torch.sort(torch.randperm(w.S, device=dev, generator=g)[:k]).values.to(torch.int32)
    Ka, Va = torch.empty(k, w.Hkv, w.D, dtype=tdt, device=dev), torch.empty(k, w.Hkv, w.D, dtype=tdt, device=dev)
    fn = lambda: dash.dash_compact_many(kept, [(K, Ka), (V, Va)])
    nbytes = k * (2.0 * 2 * w.Hkv * w.D * esz + 4.0)
    warm, cold = timed_calls(torch, fn, 10), timed_calls(torch, fn, 5, flush)
    assert torch.equal(Ka, K[kept.long()]) and torch.equal(Va, V[kept.long()])
    out["gather_kv"] = {"rows": k, "bytes": nbytes, "ms": warm, "ms_cold": cold,
                        "frac": nbytes / (warm * 1e-3) / 1e9 / PEAK_HBM_GBPS,
                        "frac_cold": nbytes / (cold * 1e-3) / 1e9 / PEAK_HBM_GBPS}
    # the same bytes as a plain device-to-device copy, for reference
    src = torch.empty(int(nbytes) // 2, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    fn = lambda: dst.copy_(src)
    warm, cold = timed_calls(torch, fn, 10), timed_calls(torch, fn, 5, flush)
    out["device_copy_same_bytes"] = {"ms": warm, "ms_cold": cold,
                                     "frac": nbytes / (warm * 1e-3) / 1e9 / PEAK_HBM_GBPS,
                                     "frac_cold": nbytes / (cold * 1e-3) / 1e9 / PEAK_HBM_GBPS}
    if args.calibrate_copy:
        a = torch.empty(512 << 20, dtype=torch.uint8, device=dev).fill_(1)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
    print(json.dumps(out), flush=True)


def score_measurements(dash, torch, dev, step, layer):
    """The score two ways on the scored full-length layer: standalone
    (||U_t|| read back from a stored U: hidden * element size B read + 4 B
    written per row, HBM bound) and fused (the W_o GEMM with and without the
    sum of squares)."""
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
        for _ in range(3):
            dash.dash_attn_layer(layer.Q, layer.K, layer.V, layer.Wo, step.O, step.U,
                                 step.score if with_score else None, ws)
        dash.trace_stop()
        proj.setdefault(with_score, []).extend(ms for op, ms in dash.trace_read(64) if op == "proj_layer")
    with_ms = sum(proj[True]) / len(proj[True])
    without_ms = sum(proj[False]) / len(proj[False])
    out.update({"fused_proj_us": with_ms * 1e3, "plain_proj_us": without_ms * 1e3,
                "fused_overhead_us": (with_ms - without_ms) * 1e3})
    return out


def decode_measurements(dash, torch, dev, w, layer, k):
    """One decode token per sample against the cache a prefill leaves: the k kept
    rows (pruned) versus all S rows (dense), same kernels; the cache read (K and
    V of every cached row) is the algorithmic traffic.  A decode loop issues
    many small launches, so the calls are captured in a HIP graph (20 calls)
    and timed by replaying it on a busy GPU; each replay's output is checked
    against the eager call's."""
    res = {}
    Hkv, D, Hq = w.Hkv, w.D, w.Hq
    Qd = layer.Q[:1].reshape(1, 1, Hq, D).contiguous()
    for name, rows in (("pruned", k), ("dense", w.S)):  # cache rows, the new token's own included
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


def describe(w, step):
    s = (f"{w.name}: S={w.S}, Hq={w.Hq}, Hkv={w.Hkv}, D={w.D}, hidden={w.hidden}, {w.layers} layers, ")
    if w.mode == "threshold":
        return s + (f"threshold halting (tau = {w.tau_pct}th-percentile layer-0 score, patience {w.patience}), "
                    f"kv_mode={w.kv_mode}")
    return s + f"one-shot halt at layer {w.halt_layer}, top-k keep {w.keep} (k={step.k}), kv_mode={w.kv_mode}" + (
        ", clustered salience" if w.clustered else "")


def active_sets(step):
    """Active query positions of each post-halt layer of the last threshold run (host copies)."""
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


def blas_info():
    try:
        from threadpoolctl import threadpool_info
        for i in threadpool_info():
            if i.get("user_api") == "blas":
                return {"vendor": i.get("internal_api"), "version": i.get("version"),
                        "threads": int(i.get("num_threads", 1))}
    except Exception:  # noqa: BLE001 - report what is known
        pass
    return {"vendor": None, "version": None, "threads": 1}


def cpu_baseline(w, host_keep, step, k_rows):
    """The CPU oracle (float64 NumPy, as it stands) on the same seeded inputs.

    Short sequences: whole steps.  Long ones: the oracle on uniformly sampled
    blocks of 128 consecutive query rows (its own block size, so each block
    costs what it costs inside a whole-layer call) of one full-length layer and
    of one post-halt layer, scaled by the number of blocks, then by the layer
    counts (labelled extrapolated)."""
    import oracle
    blas = blas_info()
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        affinity = os.cpu_count()
    base = {"unit": "tokens/s", "cores": blas["threads"], "kind": "oracle", "affinity_cores": affinity,
            "blas": blas}
    if w.S <= 8192:
        # whole steps (halting layer at full length + top-k + post-halt layer(s)), repeated until
        # about 10 s of CPU work has been timed (at most 4 repetitions)
        k = oracle.topk_count(w.S, w.keep)
        reps, t = 0, 0.0
        while reps < 4 and (reps == 0 or t < 10.0):
            t0 = time.perf_counter()
            x = host_keep[w.halt_layer]
            _, _, s = oracle.attention_layer(x["Q"], x["K"], x["V"], x["Wo"])
            idx = oracle.select_topk(s, k)
            for l in range(w.halt_layer + 1, w.layers):
                y = host_keep[l]
                oa = oracle.attn_active(y["Q"], y["K"], y["V"], idx, w.kv_mode)
                oracle.output_projection(oa, y["Wo"])
            t += time.perf_counter() - t0
            reps += 1
        per = t / reps
        sample = (f"{reps} whole step(s) of the same seeded workload (halt layer at full length + top-k + "
                  f"{w.layers - w.halt_layer - 1} post-halt layer), float64, {t:.1f} s in total")
        return dict(base, value=w.S / per, sample=sample, seconds=t)
    rng = np.random.default_rng(0)
    BR = 128
    nb = 12  # sampled blocks per layer kind

    def blocks_time(Q, K, V, Wo, q_pos_all, kv_pos, n_rows):
        n_blk = (n_rows + BR - 1) // BR
        pick = np.sort(rng.choice(n_blk, min(nb, n_blk), replace=False))
        t0 = time.perf_counter()
        for b in pick:
            r = np.arange(b * BR, min(n_rows, (b + 1) * BR))
            O = oracle.causal_gqa_attention(Q[r], K, V, q_pos=q_pos_all[r], kv_pos=kv_pos)
            oracle.delta_attn(oracle.output_projection(O, Wo))
        return (time.perf_counter() - t0) * n_blk / pick.size, pick.size

    x = host_keep[w.halt_layer if w.mode != "threshold" else 0]
    t_full, b_full = blocks_time(x["Q"], x["K"], x["V"], x["Wo"], np.arange(w.S), None, w.S)
    y = host_keep[w.halt_layer + 1 if w.mode != "threshold" else 1]
    if w.mode == "threshold":
        # a post-halt layer over its active rows (kv all), the GPU run's trajectory for the counts
        n = k_rows[0]
        pos = np.sort(rng.choice(w.S, n, replace=False)) if n < w.S else np.arange(w.S)
        t_p, b_post = blocks_time(y["Q"][pos], y["K"], y["V"], y["Wo"], pos, None, n)
        est = t_full + sum(t_p * (kr / max(1, n)) for kr in k_rows)
        n_full = 1
    else:
        k = step.k
        idx = np.sort(rng.choice(w.S, k, replace=False))
        t_p, b_post = blocks_time(y["Q"][idx], y["K"][idx], y["V"][idx], y["Wo"], idx, idx, k)
        n_full = w.halt_layer + 1
        est = n_full * t_full + (w.layers - n_full) * t_p
    return dict(base, value=w.S / est,
                sample=(f"{b_full} and {b_post} uniformly sampled blocks of {BR} query rows of one full-length "
                        f"and one post-halt layer (float64), scaled to whole layers and extrapolated to the "
                        f"{w.layers}-layer stack: {est:.0f} s"),
                extrapolated=True)


if __name__ == "__main__":
    main()
