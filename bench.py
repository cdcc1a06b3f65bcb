#!/usr/bin/env python3
"""Benchmark of the KDA forward hot path on one MI355X.

One step = one chunked prefill over the main prefill workload (B1 T8192 H64
d128, bf16 q/k/v/beta, fp32 g and state, bf16 output) plus one decode step
over the decode workload (256 requests x 64 heads, 128x128 fp32 states
updated in place, bf16 output). Inputs are synthetic (seeded generators) and resident in
HBM before timing starts. Prints one JSON line. Besides the step figures it
reports the decode step repeated back to back (the sustained rate) and the
same step for Gated DeltaNet (one scalar gate per token and head) and Gated
DeltaNet-2 (erase and write gates per channel in place of beta), and the
serving-state operations (4-token verification against a slot-indexed state
pool, with and without per-token snapshots, and a 256-state fork copy), the
packed long-context prefill (8 sequences, 105,872 tokens, drawn on the device),
and the input preparation pass at the main prefill's shape.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                  [--no-extras | --extras b2b,gdn,gdn2,serving,varlen,inputs]
  python bench.py --copy-calibration          # 1 GiB device copy (counter calibration)
  python bench.py --traffic-summary F W CF CW # rocprofv3 --pmc CSVs -> profiles/ json

The traffic summary takes four rocprofv3 counter-collection CSV files: FETCH_SIZE
and WRITE_SIZE over a bench run, then over a --copy-calibration run; each counter
is scaled by the factor that makes it read 1 GiB for the copy.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
BF16_PEAK_TFLOPS = 2500.0      # dense bf16 MFMA
METRIC = "KDA prefill tokens/s (H=64,d=128,bf16) + decode-step state GB/s vs peak"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_main_prefill_and_decode.json")
COPY_BYTES = 1 << 30
KERNEL_DESC = ("kda_fwd_chunked call (prep_fast_kernel + state_kernel; packed input adds "
               "chunk_map_kernel), one launch sequence per step")


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
    """Algorithmic flops of one prefill call, 1 FMA = 2 flops, triangles counted as
    triangles: per chunk-head A_kk 2 C(C-1)/2 Dk, A_qk 2 C(C+1)/2 Dk, the forward
    substitution sum_i i(i-1), W and U C^2 Dk and C^2 Dv, the three state contractions
    6 C Dk Dv, A_qk E 2 C(C+1)/2 Dv and the state decay Dk Dv (9,020,800 at d = 128)."""
    tri, trid = C * (C - 1) // 2, C * (C + 1) // 2
    per_chunk = (2 * tri * Dk + 2 * trid * Dk + sum(i * (i - 1) for i in range(C))
                 + C * C * Dk + C * C * Dv + 6 * C * Dk * Dv + 2 * trid * Dv + Dk * Dv)
    return per_chunk * H * (T // C)


def _code_only(text: str, python: bool = False) -> str:
    """Source text without comments and blank space, so that comment edits keep the hash."""
    if python:
        text = re.sub(r"#[^\n]*", " ", text)
    else:
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernels_source_hash():
    """sha256 over the kernel sources and build script, comments and spacing removed (the
    counter figures are tied to the code they were taken on)."""
    h = hashlib.sha256()
    pkg = os.path.join(ROOT, "gated_delta_rule_channel_amd")
    files = sorted(f for f in glob.glob(os.path.join(pkg, "csrc", "*"))
                   if f.endswith((".hip", ".h", ".cpp"))) + [os.path.join(pkg, "build.py")]
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "r", encoding="utf-8", errors="replace") as fh:
            h.update(_code_only(fh.read(), python=f.endswith(".py")).encode())
    return h.hexdigest()


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# ------------------------------------------------------------------------------------------
# counter summary
# ------------------------------------------------------------------------------------------
def _pmc_per_kernel(path, counter):
    """Average value per dispatch of one counter, per kernel name, from a rocprofv3 CSV."""
    per_dispatch = {}
    with open(path) as fh:
        for r in csv.DictReader(fh):
            if r["Counter_Name"] != counter:
                continue
            key = (r["Dispatch_Id"], r["Kernel_Name"])
            per_dispatch[key] = per_dispatch.get(key, 0.0) + float(r["Counter_Value"])
    sums, counts = {}, {}
    for (_, name), v in per_dispatch.items():
        sums[name] = sums.get(name, 0.0) + v
        counts[name] = counts.get(name, 0) + 1
    return {n: (sums[n] / counts[n], counts[n]) for n in sums}


def _short(name):
    """Kernel of the KDA path a counter row belongs to; the Gated DeltaNet and Gated
    DeltaNet-2 instantiations (a true gate flag among the template arguments, "Lb1E" in a
    mangled name) and the raw-input and gated modes of the bf16 prep kernel (mode 1, 2) are
    not counted."""
    if re.search(r"\btrue\b|Lb1E", name):
        return None
    if "prep_fast_kernel" in name:
        return "prep_kernel" if re.search(r"prep_fast_kernel<0>|prep_fast_kernelILi0E", name) else None
    for key in ("prep_kernel", "state_kernel", "chunk_map_kernel", "decode_kernel"):
        if key in name:
            return key
    return None


def traffic_summary(fetch_csv, write_csv, cfetch_csv, cwrite_csv, out_file=None):
    """Per-kernel HBM bytes from two FETCH_SIZE / WRITE_SIZE passes, scaled by what the same
    counters read for a 1 GiB copy; written to out_file (the profiles JSON by default)."""
    out_file = out_file or TRAFFIC_FILE
    cf = max(v for v, _ in _pmc_per_kernel(cfetch_csv, "FETCH_SIZE").values())
    cw = max(v for v, _ in _pmc_per_kernel(cwrite_csv, "WRITE_SIZE").values())
    f_fac = COPY_BYTES / (cf * 1024.0)
    w_fac = COPY_BYTES / (cw * 1024.0)
    fetch = _pmc_per_kernel(fetch_csv, "FETCH_SIZE")
    write = _pmc_per_kernel(write_csv, "WRITE_SIZE")
    per = {}
    for name, (v, n) in fetch.items():
        s = _short(name)
        if s:
            per.setdefault(s, {})["fetch_bytes"] = v * 1024.0 * f_fac
            per[s]["dispatches"] = n
    for name, (v, n) in write.items():
        s = _short(name)
        if s:
            per.setdefault(s, {})["write_bytes"] = v * 1024.0 * w_fac
    out = {
        "kernels_source_sha256": kernels_source_hash(),
        "calibration": {"copy_bytes": COPY_BYTES, "copy_fetch_kib": cf, "copy_write_kib": cw,
                        "fetch_factor": f_fac, "write_factor": w_fac},
        "per_kernel": per,
        "prefill_call_bytes": sum(per[k]["fetch_bytes"] + per[k]["write_bytes"]
                                  for k in ("chunk_map_kernel", "prep_kernel", "state_kernel")
                                  if k in per),
        "decode_bytes": (per["decode_kernel"]["fetch_bytes"] + per["decode_kernel"]["write_bytes"]
                         if "decode_kernel" in per else None),
    }
    os.makedirs(os.path.dirname(out_file), exist_ok=True)
    with open(out_file, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out, indent=1))
    return out


def load_traffic(path=None):
    """Measured HBM bytes per prefill call and per decode step, or None when the counters
    were taken on different kernel sources."""
    path = path or TRAFFIC_FILE
    if not os.path.exists(path):
        return None, None
    try:
        d = json.load(open(path))
    except (OSError, ValueError):
        return None, None
    if d.get("kernels_source_sha256") != kernels_source_hash():
        return None, None
    return d.get("prefill_call_bytes"), d.get("decode_bytes")


# ------------------------------------------------------------------------------------------
# modes
# ------------------------------------------------------------------------------------------
def copy_calibration():
    import torch
    x = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES, "copies": 3}), flush=True)


def cpu_baseline(wp, min_seconds):
    """The float64 C oracle over all heads of the main prefill workload, repeated until at
    least min_seconds of CPU time have passed (input generation excluded)."""
    from gated_delta_rule_channel_amd import inputs as I
    from oracle import native
    native.build()
    x = I.prefill_inputs(wp)
    tokens = x.q.shape[0] * x.q.shape[1]
    passes, t0 = 0, time.perf_counter()
    while True:
        native.prefill(x.q, x.k, x.v, x.g, x.beta)
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    threads = native.num_threads()
    # one thread on 4 of the heads, scaled to the whole workload
    hs = min(4, wp.H)
    sl = [t[:, :, :hs].contiguous() for t in (x.q, x.k, x.v, x.g, x.beta)]
    native.set_num_threads(1)
    try:
        p1, t1 = 0, time.perf_counter()
        while True:
            native.prefill(*sl)
            p1 += 1
            d1 = time.perf_counter() - t1
            if d1 >= min_seconds / 3:
                break
    finally:
        native.set_num_threads(threads)
    return {"value": tokens * passes / dt, "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": f"float64 C oracle (OpenMP over heads), all {wp.H} heads of {wp.name}, "
                      f"{passes} passes in {dt:.1f} s (input cast to fp32 included)",
            "one_thread": {"value": tokens * p1 * hs / wp.H / d1, "unit": "tokens/s",
                           "sample": f"{hs} of {wp.H} heads, {p1} passes in {d1:.1f} s, "
                                     f"scaled to all heads"},
            "cpu_model": _cpu_model()}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="time only the step (prefill + decode); for counter passes")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--extras", default="all",
                    help="comma-separated sections after the step: b2b, gdn, gdn2, serving, "
                         "varlen, inputs (default all)")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--traffic-summary", nargs=4, metavar=("FETCH", "WRITE", "CFETCH", "CWRITE"))
    args = ap.parse_args()
    if args.traffic_summary:
        traffic_summary(*args.traffic_summary)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the KDA hot path here runs on a single MI355X "
              "(heads, requests and sequences shard across GPUs without exchange). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return

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
    # outputs in the input dtype (bf16), as the workloads specify; states fp32
    o = torch.empty((B, T, H, Dv), dtype=torch.bfloat16, device=dev)
    ht = torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=dev)
    od = torch.empty((wd.N, wd.H, wd.Dv), dtype=torch.bfloat16, device=dev)

    def prefill():
        kda.fwd_chunked(q, k, v, g, b, scale=1.0, workspace=ws, out=o, final_state=ht)

    def decode():
        kda.decode_step(dq, dk, dv, dg, db, state, scale=1.0, out=od)

    # both calls launch on torch's current stream, which the events below record on
    stream = torch.cuda.current_stream(dev)
    for _ in range(args.warmup):
        prefill()
        decode()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
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
    # algorithmic bytes of the hot-path table: q, k, v, beta bf16, g fp32, o bf16, ht fp32
    # (810,549,248 B here)
    pf_bytes = prefill_bytes(T, H, Dk, Dv, 2, 2, B)
    dc_bytes = decode_bytes(wd.N, wd.H, wd.Dk, wd.Dv, 2, 2)
    pf_flops = prefill_flops(T, H, Dk, Dv)
    value = tokens / tp_mean
    pf_gbs = pf_bytes / tp_mean / 1e9
    dc_gbs = dc_bytes / td_mean / 1e9
    # roofline time of the call: max(algorithmic bytes / 8 TB/s, MFMA time); with split-bf16
    # operands every product runs as three bf16 MFMAs
    t_hbm = pf_bytes / (HBM_PEAK_GBS * 1e9)
    t_mfma = 3.0 * pf_flops / (BF16_PEAK_TFLOPS * 1e12)
    t_roof = max(t_hbm, t_mfma)
    mfma_busy = t_mfma / tp_mean
    mfma_alg = pf_flops / (BF16_PEAK_TFLOPS * 1e12) / tp_mean
    traffic_pf, traffic_dc = load_traffic()

    sel = set(args.extras.split(","))

    def want(name):
        return "all" in sel or name in sel

    def run_extras():
        """The figures beyond the step: back-to-back decode, Gated DeltaNet, Gated DeltaNet-2,
        serving state, the packed long-context prefill and input preparation (the sections
        named by --extras)."""
        def timed(fn, n):
            for _ in range(3):
                fn()
            a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a0.record(stream)
            for _ in range(n):
                fn()
            a1.record(stream)
            torch.cuda.synchronize()
            return a0.elapsed_time(a1) * 1e-3 / n

        n_serv = max(5, args.steps // 2)
        res = {}

        if want("b2b"):
            # the same decode step repeated with nothing between the calls: the Infinity Cache holds
            # the tail of each step's state writes, which then reach HBM inside the next step rather
            # than under the following prefill, so this is the sustained decode rate
            eb0, eb1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            eb0.record(stream)
            for _ in range(args.steps):
                decode()
            eb1.record(stream)
            torch.cuda.synchronize()
            td_b2b = eb0.elapsed_time(eb1) * 1e-3 / args.steps
            dc_gbs_b2b = dc_bytes / td_b2b / 1e9

        if want("gdn"):
            # Gated DeltaNet (scalar gate per token and head) on the same q, k, v, beta and state
            # shapes, timed the same way (one prefill + one decode step per step)
            gs = I.scalar_gate(wp, list(range(H)), B * T).view(B, T, H).to(dev)
            gds = I.scalar_gate(wd, list(range(wd.H)), wd.N).to(dev)

            def gdn_prefill():
                kda.gdn_fwd_chunked(q, k, v, gs, b, scale=1.0, workspace=ws, out=o, final_state=ht)

            def gdn_decode():
                kda.gdn_decode_step(dq, dk, dv, gds, db, state, scale=1.0, out=od)

            for _ in range(args.warmup):
                gdn_prefill()
                gdn_decode()
            torch.cuda.synchronize()
            for e0, e1, e2 in ev:
                e0.record(stream)
                gdn_prefill()
                e1.record(stream)
                gdn_decode()
                e2.record(stream)
            torch.cuda.synchronize()
            tgp = np.array([a.elapsed_time(bb) for a, bb, _ in ev]) * 1e-3
            tgd = np.array([bb.elapsed_time(c) for _, bb, c in ev]) * 1e-3
            gdn_pf_bytes = pf_bytes - B * T * H * Dk * 4 + B * T * H * 4       # g is one float per token-head
            gdn_dc_bytes = dc_bytes - wd.N * wd.H * wd.Dk * 4 + wd.N * wd.H * 4

        if want("gdn2"):
            # Gated DeltaNet-2 (erase gate per key channel, write gate per value channel, bf16, in
            # place of beta) on the same q, k, v, g and state, timed the same way
            eb2, ew2 = (t.view(B, T, H, -1).to(dev) for t in I.erase_write_gates(wp, list(range(H)), B * T))
            ebd, ewd = (t.to(dev) for t in I.erase_write_gates(wd, list(range(wd.H)), wd.N))

            def gdn2_prefill():
                kda.gdn2_fwd_chunked(q, k, v, g, eb2, ew2, scale=1.0, workspace=ws, out=o, final_state=ht)

            def gdn2_decode():
                kda.gdn2_decode_step(dq, dk, dv, dg, ebd, ewd, state, scale=1.0, out=od)

            for _ in range(args.warmup):
                gdn2_prefill()
                gdn2_decode()
            torch.cuda.synchronize()
            for e0, e1, e2 in ev:
                e0.record(stream)
                gdn2_prefill()
                e1.record(stream)
                gdn2_decode()
                e2.record(stream)
            torch.cuda.synchronize()
            t2p = np.array([a.elapsed_time(bb) for a, bb, _ in ev]) * 1e-3
            t2d = np.array([bb.elapsed_time(c) for _, bb, c in ev]) * 1e-3
            del eb2, ew2
            gdn2_pf_bytes = pf_bytes - B * T * H * 2 + B * T * H * (Dk + Dv) * 2   # b, w instead of beta
            gdn2_dc_bytes = dc_bytes - wd.N * wd.H * 2 + wd.N * wd.H * (wd.Dk + wd.Dv) * 2

        if want("serving"):
            # serving state: 4 drafted tokens per request verified against a pool of 512 slots (the
            # 256 requests at permuted slots), without and with per-token snapshots, and a fork of
            # 256 states to free slots
            TV, PS = 4, 2 * wd.N
            xs = I.decode_inputs(wd, N=wd.N * TV, with_state=False)
            mv = [t.view(wd.N, TV, *t.shape[1:]).to(dev) for t in (xs.q, xs.k, xs.v, xs.g, xs.beta)]
            del xs
            spool = torch.empty((PS, wd.H, wd.Dk, wd.Dv), dtype=torch.float32, device=dev)
            spool[:wd.N].copy_(state)
            spool[wd.N:].copy_(state)
            perm = np.random.default_rng(5).permutation(PS).astype(np.int32)
            sslots = torch.from_numpy(perm[:wd.N]).to(dev)
            fork_src = torch.from_numpy(perm[:wd.N]).to(dev)
            fork_dst = torch.from_numpy(perm[wd.N:]).to(dev)
            snaps = torch.empty((wd.N, TV, wd.H, wd.Dk, wd.Dv), dtype=torch.float32, device=dev)
            omv = torch.empty((wd.N, TV, wd.H, wd.Dv), dtype=torch.bfloat16, device=dev)


            t_mv = timed(lambda: kda.decode_multi(*mv, spool, slots=sslots, scale=1.0, out=omv), n_serv)
            t_mvs = timed(lambda: kda.decode_multi(*mv, spool, slots=sslots, snapshots=snaps, scale=1.0,
                                                   out=omv), n_serv)
            t_fork = timed(lambda: kda.state_copy(spool, fork_dst, spool, fork_src), n_serv)
            st_bytes = wd.N * wd.H * wd.Dk * wd.Dv * 4
            tok_bytes = TV * (decode_bytes(wd.N, wd.H, wd.Dk, wd.Dv, 2, 2) - 2 * st_bytes)
            mv_bytes = 2 * st_bytes + tok_bytes
            mvs_bytes = mv_bytes + TV * st_bytes
            del spool, snaps, mv, omv

        if want("varlen"):
            # the packed long-context workload: 8 sequences of the seeded lengths (105,872 tokens),
            # H64 d128 bf16, drawn on the device with the generators' distributions (unit q, k with q
            # scaled by d^-1/2, v ~ N(0, 1), beta = sigmoid(N(0, 1)), g = -softplus(N(0, 1)) U(0.5, 2)
            # with 13 fast channels at -U(5, 10) and 13 slow ones at -U(0, 1e-4) per head)
            wv = I.WORKLOADS[4]
            lens = I.varlen_lengths(wv)
            cu_v = torch.from_numpy(I.cu_seqlens_from_lengths(lens)).to(dev)
            TV_ = int(lens.sum())
            gv = torch.Generator(device=dev).manual_seed(4)
            rn = lambda *shape: torch.randn(shape, generator=gv, device=dev)
            unit = lambda x: x / x.norm(dim=-1, keepdim=True)
            vq = (unit(rn(1, TV_, H, Dk)) * Dk ** -0.5).to(torch.bfloat16)
            vk = unit(rn(1, TV_, H, Dk)).to(torch.bfloat16)
            vv = rn(1, TV_, H, Dv).to(torch.bfloat16)
            vb = torch.sigmoid(rn(1, TV_, H)).to(torch.bfloat16)
            vg = -torch.nn.functional.softplus(rn(1, TV_, H, Dk))
            vg *= torch.empty_like(vg).uniform_(0.5, 2.0, generator=gv)
            for h in range(H):
                perm = torch.randperm(Dk, generator=gv, device=dev)
                fast, slow = perm[:13], perm[13:26]
                vg[0, :, h, fast] = -torch.empty((TV_, 13), device=dev).uniform_(5.0, 10.0, generator=gv)
                vg[0, :, h, slow] = -torch.empty((TV_, 13), device=dev).uniform_(0.0, 1e-4, generator=gv)
            nbv = kda.workspace_size(1, TV_, H, Dk, Dv, len(lens), True, kda.KDA_DTYPE_BF16)
            wsv = torch.empty(nbv, dtype=torch.uint8, device=dev)
            ov = torch.empty((1, TV_, H, Dv), dtype=torch.bfloat16, device=dev)
            htv = torch.empty((len(lens), H, Dk, Dv), dtype=torch.float32, device=dev)
            t_var = timed(lambda: kda.fwd_chunked(vq, vk, vv, vg, vb, cu_seqlens=cu_v, workspace=wsv,
                                                  out=ov, final_state=htv), max(3, n_serv // 5))
            # algorithmic bytes per token as for the main prefill (bf16 o): 98,432 at H64 d128
            var_bytes = TV_ * H * (3 * Dk * 2 + Dk * 4 + 2 + Dv * 2) + len(lens) * H * Dk * Dv * 4
            del vq, vk, vv, vb, vg, wsv, ov, htv

        if want("inputs"):
            # input preparation at the main prefill's shape: raw bf16 q, k, a [T, H, Dk] and b [T, H]
            # to normalised q, k (bf16), g (fp32) and beta (bf16), one pass
            rng_i = torch.Generator(device=dev).manual_seed(3)
            raw = [torch.randn((B * T, H, Dk), generator=rng_i, device=dev).to(torch.bfloat16)
                   for _ in range(3)]
            raw.append(torch.randn((B * T, H), generator=rng_i, device=dev).to(torch.bfloat16))
            prep_out = (torch.empty_like(raw[0]), torch.empty_like(raw[1]),
                        torch.empty((B * T, H, Dk), dtype=torch.float32, device=dev),
                        torch.empty_like(raw[3]))
            t_prep = timed(lambda: kda.prepare_inputs(*raw, scale=Dk ** -0.5, out=prep_out), n_serv)
            prep_bytes = B * T * H * (Dk * 2 * 5 + Dk * 4 + 2 * 2)
            # raw projections to o at the main prefill's shape: the two-pass route (the preparation
            # above, then the prefill on its outputs) against kda_fwd_chunked_raw, which forms the
            # prepared inputs inside the prefill's first kernel
            rs = lambda t: t.view(B, T, *t.shape[1:])
            p4 = [rs(t) for t in prep_out]

            def two_pass():
                kda.prepare_inputs(*raw, scale=Dk ** -0.5, out=prep_out)
                kda.fwd_chunked(p4[0], p4[1], v, p4[2], p4[3], scale=1.0, workspace=ws, out=o,
                                final_state=ht)

            r4 = [rs(t) for t in raw]
            # the main prefill with a float32 o instead of the input dtype (2 more bytes per output
            # element), for comparison
            o32 = torch.empty((B, T, H, Dv), dtype=torch.float32, device=dev)
            t_o32 = timed(lambda: kda.fwd_chunked(q, k, v, g, b, scale=1.0, workspace=ws, out=o32,
                                                  final_state=ht), n_serv)
            del o32
            t_two = timed(two_pass, n_serv)
            t_raw = timed(lambda: kda.fwd_chunked_raw(r4[0], r4[1], v, r4[2], r4[3], scale=Dk ** -0.5,
                                                      workspace=ws, out=o, final_state=ht), n_serv)
            del raw, prep_out, p4, r4
        if want("b2b"):
            res["decode_b2b"] = {"ms_back_to_back": td_b2b * 1e3, "hbm_gbs_back_to_back": dc_gbs_b2b,
                                 "frac_of_peak_back_to_back": dc_gbs_b2b / HBM_PEAK_GBS}
        if want("gdn"):
            res["gated_deltanet"] = {"prefill_ms": float(tgp.mean()) * 1e3,
                                     "prefill_tokens_per_s": tokens / float(tgp.mean()),
                                     "prefill_hbm_gbs": gdn_pf_bytes / float(tgp.mean()) / 1e9,
                                     "decode_ms": float(tgd.mean()) * 1e3,
                                     "decode_hbm_gbs": gdn_dc_bytes / float(tgd.mean()) / 1e9,
                                     "decode_frac_of_peak": gdn_dc_bytes / float(tgd.mean()) / 1e9
                                     / HBM_PEAK_GBS}
        if want("gdn2"):
            res["gated_deltanet_2"] = {"prefill_ms": float(t2p.mean()) * 1e3,
                                       "prefill_tokens_per_s": tokens / float(t2p.mean()),
                                       "prefill_hbm_gbs": gdn2_pf_bytes / float(t2p.mean()) / 1e9,
                                       "decode_ms": float(t2d.mean()) * 1e3,
                                       "decode_hbm_gbs": gdn2_dc_bytes / float(t2d.mean()) / 1e9,
                                       "decode_frac_of_peak": gdn2_dc_bytes / float(t2d.mean()) / 1e9
                                       / HBM_PEAK_GBS}
        if want("serving"):
            res["serving"] = {"verify_tokens": TV, "pool_slots": PS,
                              "decode_multi_ms": t_mv * 1e3, "decode_multi_tokens_per_s": wd.N * TV / t_mv,
                              "decode_multi_hbm_gbs": mv_bytes / t_mv / 1e9,
                              "decode_multi_snapshots_ms": t_mvs * 1e3,
                              "decode_multi_snapshots_hbm_gbs": mvs_bytes / t_mvs / 1e9,
                              "state_copy_256_ms": t_fork * 1e3,
                              "state_copy_hbm_gbs": 2 * st_bytes / t_fork / 1e9}
        if want("varlen"):
            res["varlen_prefill"] = {"workload": wv.name, "tokens": TV_, "sequences": len(lens),
                                     "ms": t_var * 1e3, "tokens_per_s": TV_ / t_var,
                                     "compulsory_bytes": var_bytes, "hbm_gbs": var_bytes / t_var / 1e9,
                                     "frac_of_peak": var_bytes / t_var / 1e9 / HBM_PEAK_GBS}
        if want("inputs"):
            res["input_prep"] = {"ms": t_prep * 1e3, "bytes": prep_bytes,
                                 "hbm_gbs": prep_bytes / t_prep / 1e9,
                                 "frac_of_peak": prep_bytes / t_prep / 1e9 / HBM_PEAK_GBS}
        if want("inputs"):
            res["prefill_fp32_o"] = {"ms": t_o32 * 1e3, "tokens_per_s": tokens / t_o32}
        if want("inputs"):
            res["raw_to_o"] = {"two_pass_ms": t_two * 1e3, "fused_ms": t_raw * 1e3,
                               "fused_tokens_per_s": tokens / t_raw,
                               "saved_ms": (t_two - t_raw) * 1e3}
        return res

    extra = {} if args.no_extras else run_extras()

    # context for the decode figure: torch's device-to-device copy of 1 GiB (read + write)
    xc = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    yc = torch.empty_like(xc)
    yc.copy_(xc)
    tc = []
    for _ in range(5):
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record(stream)
        yc.copy_(xc)
        c1.record(stream)
        torch.cuda.synchronize()
        tc.append(c0.elapsed_time(c1) * 1e-3)
    copy_gbs = 2 * COPY_BYTES / float(np.median(tc)) / 1e9
    del xc, yc

    cpu = None if args.no_cpu_baseline else cpu_baseline(wp, args.cpu_seconds)

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
        "config": {"workload": f"{wp.name} (fp32 state, bf16 o) + {wd.name} (bf16 o)",
                   "global_batch": B, "seq_len": T, "heads": H, "d_k": Dk, "d_v": Dv,
                   "chunk": 64, "parallelism": "single GPU"},
        "prefill": {"ms": tp_mean * 1e3, "ms_median": float(np.median(tp)) * 1e3,
                    "ms_min": float(tp.min()) * 1e3, "tokens_per_s": value,
                    "compulsory_bytes": pf_bytes,
                    "hbm_gbs": pf_gbs,
                    "algorithmic_flops": pf_flops, "tflops": pf_flops / tp_mean / 1e12,
                    "t_roof_us": t_roof * 1e6, "t_hbm_us": t_hbm * 1e6, "t_mfma_us": t_mfma * 1e6,
                    "frac_of_roofline": t_roof / tp_mean,
                    "mfma_busy_frac_split_bf16": mfma_busy,
                    "mfma_frac_algorithmic_flops": mfma_alg},
        "decode": {"ms": td_mean * 1e3, "ms_median": float(np.median(td)) * 1e3,
                   "ms_min": float(td.min()) * 1e3,
                   "state_updates_per_s": wd.N * wd.H / td_mean, "tokens_per_s": wd.N / td_mean,
                   "compulsory_bytes": dc_bytes, "hbm_gbs": dc_gbs,
                   "frac_of_peak": dc_gbs / HBM_PEAK_GBS,
                   "device_copy_gbs": copy_gbs, "frac_of_device_copy": dc_gbs / copy_gbs,
                   **extra.get("decode_b2b", {})},
        **{k: v for k, v in extra.items() if k != "decode_b2b"},
        "roofline": {"bound": "hbm", "achieved": pf_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": pf_gbs / HBM_PEAK_GBS, "traffic": traffic_pf,
                     "byte_basis": "algorithmic: q, k, v, beta bf16 + g fp32 + o bf16 + ht fp32 "
                                   f"= {pf_bytes} B per call",
                     "kernel": KERNEL_DESC},
        "roofline_decode": {"bound": "hbm", "achieved": dc_gbs, "peak": HBM_PEAK_GBS,
                            "unit": "GB/s", "frac": dc_gbs / HBM_PEAK_GBS, "traffic": traffic_dc,
                            "kernel": "decode_kernel"},
        "cpu_baseline": cpu,
        "wall_s_timed": t_wall,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
