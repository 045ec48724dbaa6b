#!/usr/bin/env python3
"""Benchmark of the DASH prefill hot path on one MI355X.

One step = one pass of the whole path over one synthetic sequence: the halting
layer at full length (causal GQA attention + W_o GEMM with the fused Δattn
score), top-k selection, compaction of the next layer's Q/K/V at the kept
positions, and the post-halt layer on the kept rows (attention + W_o).  The
default workload is Qwen2.5-7B-shaped: S=8192, 28 q-heads / 4 kv-heads,
head_dim 128, hidden 3584, bf16, keep ratio 0.5, kv_mode=active.

Prints one JSON line: prefill tokens/s of the step, the dense (no halting)
comparison, a roofline entry for the dominant kernel (the attention kernel,
from HIP events recorded by the library on its launch stream), per-kernel
timings, and the CPU oracle timed on this host as a reported baseline.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "prefill tokens/s (halt + post-halt layers) vs dense; attn MFMA util; select GB/s"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0     # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=1, choices=[0, 1])
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--profile-only", action="store_true",
                    help="run warmup + timed steps only (for rocprofv3); print the JSON line without the CPU leg")
    return ap.parse_args()


def attn_flops(D, Hq, n):
    """Algorithmic flops of causal attention over n rows: 4*D*Hq per (query, visible key) pair."""
    return 4.0 * D * Hq * n * (n + 1) / 2.0


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on exactly one GPU; --gpus must be 1",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)

    import torch
    import attention_delta_token_amd as dash
    from attention_delta_token_amd.stack import DenseStack, LayerTensors, OneShotStack
    from workload import WORKLOADS, layer_inputs

    dash.load()
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    w = WORKLOADS[args.config]
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    hostl = [layer_inputs(w, args.seed, l) for l in range(w.layers)]
    layers = [LayerTensors(*(torch.from_numpy(h[n]).to(dev, tdt) for n in ("Q", "K", "V")),
                           torch.from_numpy(np.ascontiguousarray(h["Wo"].T)).to(dev, tdt)) for h in hostl]
    k = w.k
    step = OneShotStack(layers, halt_layer=w.halt_layer, k=k)

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

    for _ in range(args.warmup):
        step.run()
    ms = timed(step.run, args.steps)

    # Same steps again with the library's per-launch HIP events (on the launch stream).
    dash.trace_start(64 * args.steps)
    ms_traced = timed(step.run, args.steps)
    dash.trace_stop()
    recs = dash.trace_read(64 * args.steps)

    dense_ms = None
    if not args.no_dense and not args.profile_only:
        dense = DenseStack(layers)
        for _ in range(args.warmup):
            dense.run()
        dense_ms = timed(dense.run, args.steps)

    S, Hq, Hkv, D, hid = w.S, w.Hq, w.Hkv, w.D, w.hidden
    n_full = w.halt_layer + 1
    n_post = w.layers - n_full
    by = {}
    for op, t in recs:
        by.setdefault(op, []).append(t)
    # attention kernel: full-length launches and post-halt launches (kv active: k rows)
    f_full, f_post = attn_flops(D, Hq, S), attn_flops(D, Hq, k)
    t_full, t_post = by.get("attn_layer", []), by.get("attn_active", [])
    attn_launches = len(t_full) + len(t_post)
    attn_flops_total = f_full * len(t_full) + f_post * len(t_post)
    attn_ms_total = sum(t_full) + sum(t_post)
    attn_tflops = attn_flops_total / (attn_ms_total * 1e-3) / 1e12
    avg_launch_ms = attn_ms_total / max(1, attn_launches)

    def avg(op):
        v = by.get(op, [])
        return (sum(v) / len(v)) if v else None

    proj_f_full = 2.0 * S * (Hq * D) * hid
    proj_f_post = 2.0 * k * (Hq * D) * hid
    t_pl, t_pa = by.get("proj_layer", []), by.get("proj_active", [])
    proj_tflops = ((proj_f_full * len(t_pl) + proj_f_post * len(t_pa)) /
                   ((sum(t_pl) + sum(t_pa)) * 1e-3) / 1e12) if (t_pl or t_pa) else None
    sel_bytes = 4.0 * S + 4.0 * k
    esz = 2 if w.dtype == "bf16" else 4
    compact_bytes_per_step = n_post * k * (2 * esz * (Hq * D + 2 * Hkv * D) + 3 * 4)
    n_compact_per_step = 3 * n_post
    t_sel, t_cmp = by.get("select", []), by.get("compact", [])
    sel_gbps = sel_bytes / (avg("select") * 1e-3) / 1e9 if t_sel else None
    cmp_gbps = (compact_bytes_per_step / n_compact_per_step) / (avg("compact") * 1e-3) / 1e9 if t_cmp else None

    dense_flops = w.layers * (attn_flops(D, Hq, S) + proj_f_full)
    dash_flops = n_full * (attn_flops(D, Hq, S) + proj_f_full) + n_post * (attn_flops(D, Hq, k) + proj_f_post)

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
        "config": {"workload": f"{w.name}: S={S}, Hq={Hq}, Hkv={Hkv}, D={D}, hidden={hid}, {w.layers} layers "
                               f"(halt at {w.halt_layer}), top-k keep {w.keep} (k={k}), kv_mode={w.kv_mode}",
                   "global_batch": 1, "seq_len": S, "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "kernel": "attn_fwd_bf16_kernel<128>" if D == 128 else "attn_fwd",
                     "achieved": attn_tflops, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": attn_tflops / PEAK_BF16_TFLOPS, "traffic": None,
                     "launches": attn_launches, "avg_launch_ms": avg_launch_ms,
                     "flops_per_launch_avg": attn_flops_total / max(1, attn_launches)},
        "dense_ms_per_step": dense_ms,
        "dense_tokens_per_s": (S / (dense_ms * 1e-3)) if dense_ms else None,
        "speedup_vs_dense": (dense_ms / ms) if dense_ms else None,
        "ideal_speedup_flops": dense_flops / dash_flops,
        "traced_ms_per_step": ms_traced,
        "kernels": {
            "attn_full_ms": avg("attn_layer"), "attn_post_ms": avg("attn_active"),
            "attn_full_tflops": (f_full / (avg("attn_layer") * 1e-3) / 1e12) if t_full else None,
            "attn_post_tflops": (f_post / (avg("attn_active") * 1e-3) / 1e12) if t_post else None,
            "proj_full_ms": avg("proj_layer"), "proj_post_ms": avg("proj_active"),
            "proj_tflops": proj_tflops, "proj_frac": (proj_tflops / PEAK_BF16_TFLOPS) if proj_tflops else None,
            "select_ms": avg("select"), "select_GBps": sel_gbps,
            "compact_ms": avg("compact"), "compact_GBps": cmp_gbps,
            "compact_frac": (cmp_gbps / PEAK_HBM_GBPS) if cmp_gbps else None,
        },
        "cpu_baseline": None,
    }

    if not args.no_cpu_baseline and not args.profile_only:
        out["cpu_baseline"] = cpu_baseline(w, hostl, k)

    print(json.dumps(out), flush=True)


def cpu_baseline(w, hostl, k):
    """The CPU oracle (float64 NumPy, as it stands) on one whole step of the same workload."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    t0 = time.perf_counter()
    x = hostl[w.halt_layer]
    _, _, s = oracle.attention_layer(x["Q"], x["K"], x["V"], x["Wo"])
    idx = oracle.select_topk(s, k)
    for l in range(w.halt_layer + 1, w.layers):
        y = hostl[l]
        oa = oracle.attn_active(y["Q"], y["K"], y["V"], idx, w.kv_mode)
        oracle.output_projection(oa, y["Wo"])
    t = time.perf_counter() - t0
    return {"value": w.S / t, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"one whole step ({w.layers} layers: halt layer at full length + top-k + post-halt layer) "
                      f"of the same seeded workload, float64, {t:.1f} s",
            "seconds": t}


if __name__ == "__main__":
    main()
