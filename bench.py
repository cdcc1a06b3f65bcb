#!/usr/bin/env python3
"""Benchmark of the KDA forward hot path on one MI355X.

One step = one chunked prefill over the main prefill workload (B1 T8192 H64
d128, bf16 inputs, fp32 state, fp32 output) plus one decode step over the
decode workload (256 requests x 64 heads, 128x128 fp32 states updated in
place). Inputs are synthetic (seeded generators) and resident in HBM before
timing starts. Prints one JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
BF16_PEAK_TFLOPS = 2500.0      # dense bf16 MFMA
METRIC = "KDA prefill tokens/s (H=64,d=128,bf16) + decode-step state GB/s vs peak"


def prefill_bytes(T, H, Dk, Dv, in_bytes, out_bytes, n_seq):
    """Compulsory HBM bytes of one prefill call: q, k, v, beta in, g fp32 in, o out, ht out."""
    return (T * H * (2 * Dk + Dv) * in_bytes + T * H * in_bytes + T * H * Dk * 4
            + T * H * Dv * out_bytes + n_seq * H * Dk * Dv * 4)


def decode_bytes(N, H, Dk, Dv, in_bytes, out_bytes):
    """Compulsory HBM bytes of one decode step: the state read and written once, plus
    q, k, v, beta in, g fp32 in and o out."""
    return (2 * N * H * Dk * Dv * 4 + N * H * (2 * Dk + Dv) * in_bytes + N * H * in_bytes
            + N * H * Dk * 4 + N * H * Dv * out_bytes)


def prefill_flops(T, H, Dk, Dv, C=64):
    """Algorithmic flops per chunk-head (1 FMA = 2 flops, triangles as triangles)."""
    tri = C * (C - 1) // 2          # strictly lower pairs
    trid = C * (C + 1) // 2         # lower incl. diagonal
    akk = 2 * tri * Dk + tri        # + beta scaling
    aqk = 2 * trid * Dk
    ut = sum(2 * i * (i - 1) // 2 for i in range(C))   # forward substitution
    w = 2 * trid * Dk + C * Dk
    u = 2 * trid * Dv + C * Dv
    state = 3 * 2 * C * Dk * Dv
    aqe = 2 * trid * Dv
    decay = Dk * Dv
    per_chunk = akk + aqk + ut + w + u + state + aqe + decay
    return per_chunk * H * (T // C)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=16)
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the KDA hot path here runs on a single MI355X "
              "(per-head and per-request work shards without exchange; see DESIGN.md). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import gated_delta_rule_channel_amd as kda
    from gated_delta_rule_channel_amd import inputs as I

    dev = torch.device("cuda:0")
    wp, wd = I.WORKLOADS[2], I.WORKLOADS[3]
    xp = I.prefill_inputs(wp)
    xd = I.decode_inputs(wd)
    q, k, v, g, b = (t.to(dev) for t in (xp.q, xp.k, xp.v, xp.g, xp.beta))
    dq, dk, dv, dg, db = (t.to(dev) for t in (xd.q, xd.k, xd.v, xd.g, xd.beta))
    state = xd.state.to(dev)
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    nbytes = kda.workspace_size(B, T, H, Dk, Dv, B, False, kda.KDA_DTYPE_BF16)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    o = torch.empty((B, T, H, Dv), dtype=torch.float32, device=dev)
    ht = torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=dev)
    od = torch.empty((wd.N, wd.H, wd.Dv), dtype=torch.float32, device=dev)

    def prefill():
        kda.fwd_chunked(q, k, v, g, b, scale=1.0, workspace=ws, out=o, final_state=ht)

    def decode():
        kda.decode_step(dq, dk, dv, dg, db, state, scale=1.0, out=od)

    stream = torch.cuda.current_stream(dev)
    for _ in range(args.warmup):
        prefill()
        decode()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t_wall0 = time.perf_counter()
    for e0, e1, e2 in ev:
        e0.record(stream)
        prefill()
        e1.record(stream)
        decode()
        e2.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall0
    tp = np.array([a.elapsed_time(bb) for a, bb, _ in ev]) * 1e-3   # seconds
    td = np.array([bb.elapsed_time(c) for _, bb, c in ev]) * 1e-3
    tp_mean, td_mean = float(tp.mean()), float(td.mean())

    tokens = B * T
    pf_bytes = prefill_bytes(T, H, Dk, Dv, 2, 4, B)
    dc_bytes = decode_bytes(wd.N, wd.H, wd.Dk, wd.Dv, 2, 4)
    pf_flops = prefill_flops(T, H, Dk, Dv)
    value = tokens / tp_mean
    pf_gbs = pf_bytes / tp_mean / 1e9
    dc_gbs = dc_bytes / td_mean / 1e9

    traffic = None
    tfile = os.path.join(ROOT, "profiles", "prefill_main_traffic.json")
    if os.path.exists(tfile):
        try:
            traffic = json.load(open(tfile)).get("bytes_per_call")
        except Exception:
            traffic = None

    cpu = None
    if not args.no_cpu_baseline:
        from oracle import native
        hs = list(range(min(args.cpu_heads, H)))
        xs = I.prefill_inputs(wp, heads=hs)
        native.build()
        t0 = time.perf_counter()
        native.prefill(xs.q, xs.k, xs.v, xs.g, xs.beta)
        dt = time.perf_counter() - t0
        cpu = {"value": tokens * len(hs) / H / dt, "unit": "tokens/s", "cores": native.num_threads(),
               "kind": "oracle",
               "sample": f"float64 C oracle (OpenMP over heads) on {len(hs)} of {H} heads of the "
                         f"main prefill workload (T={T}), {dt:.2f} s; tokens/s scaled to all {H} heads",
               "cpu_model": platform.processor() or _cpu_model()}

    out = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": (tp_mean + td_mean) * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{wp.name} (fp32 state, fp32 o) + {wd.name}",
                   "global_batch": B, "seq_len": T, "heads": H, "d_k": Dk, "d_v": Dv,
                   "chunk": 64, "parallelism": "single GPU"},
        "prefill": {"ms": tp_mean * 1e3, "ms_min": float(tp.min()) * 1e3, "tokens_per_s": value,
                    "compulsory_bytes": pf_bytes, "hbm_gbs": pf_gbs,
                    "algorithmic_flops": pf_flops, "tflops": pf_flops / tp_mean / 1e12},
        "decode": {"ms": td_mean * 1e3, "ms_min": float(td.min()) * 1e3,
                   "state_updates_per_s": wd.N * wd.H / td_mean, "tokens_per_s": wd.N / td_mean,
                   "compulsory_bytes": dc_bytes, "hbm_gbs": dc_gbs,
                   "frac_of_peak": dc_gbs / HBM_PEAK_GBS},
        "roofline": {"bound": "hbm", "achieved": pf_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": pf_gbs / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": "kda_fwd_chunked (chunk map + prep + state pass) per call"},
        "roofline_decode": {"bound": "hbm", "achieved": dc_gbs, "peak": HBM_PEAK_GBS,
                            "unit": "GB/s", "frac": dc_gbs / HBM_PEAK_GBS,
                            "kernel": "decode_kernel"},
        "cpu_baseline": cpu,
        "wall_s_timed": t_wall,
    }
    print(json.dumps(out), flush=True)


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


if __name__ == "__main__":
    main()
