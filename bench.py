#!/usr/bin/env python3
"""Benchmark of the gfx950 selective scan (one GPU).

One step = one forward selective scan (ssm_scan_fwd: discretisation, scan,
readout, D skip, SiLU gate, last_state) over a mamba-2.8b-shaped layer:
batch 4, seqlen 8192, d_inner 5120, d_state 16, bf16 x/delta/z/B/C, fp32
A/D/bias/state.  Inputs are seeded synthetic tensors already resident in HBM.

Prints one JSON line:  value = B*T*D elements per second (wall clock over the
timed steps), plus the roofline of the scan kernel (HIP events on the stream
the kernel runs on) and the fp64 CPU oracle timed on a bounded sample of the
same workload.

    python bench.py [--steps K] [--warmup W] [--workload 0..4] [--extra]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E
N_CU, CLOCK_HZ, LANES_PER_CU = 256, 2.4e9, 64   # 4 SIMD x 16 lanes, plain fp32 VALU


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_bytes(w, io_bytes, with_last=True):
    """Bytes the method must move once: x, delta, z read + y written per
    element; B, C per (b, t, n); A, D, bias per channel; h0 / last_state."""
    Bt, T, Dd, N = w.batch, w.seqlen, w.d_inner, w.d_state
    b = 4 * Bt * T * Dd * io_bytes            # x, delta, z, y
    b += 2 * Bt * T * N * io_bytes            # B, C
    b += (Dd * N + 2 * Dd) * 4                # A, D, delta_bias
    if w.h0_kind != "none":
        b += Bt * Dd * N * 4
    if with_last:
        b += Bt * Dd * N * 4
    return b


def source_hash(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


SCAN_SOURCES = ["selective_scan_ssm_amd/csrc/scan_fwd.hip", "selective_scan_ssm_amd/csrc/ssm_device.h"]


def traffic_from_profile(kernel_files, name):
    """HBM bytes per launch measured by rocprofv3 (FETCH_SIZE + WRITE_SIZE,
    scaled by the copy-kernel factor), if the stored measurement was taken on
    the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{name}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("source_hash") != source_hash(kernel_files):
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(inp, w, seconds_target):
    """The fp64 oracle on a bounded sample of the workload: all batches and the
    first `nd` channels over the full sequence."""
    import numpy as np
    import oracle
    from selective_scan_ssm_amd import inputs as gen
    io = inp["io"]
    threads = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    threads = max(1, min(16, threads))
    # oracle speed is about 7e6 elements/s per core at d_state 16: size the
    # sample to roughly `seconds_target` core-seconds of work
    per_core = 7e6 * 16 / max(1, w.d_state)
    nd = int(min(w.d_inner, max(64, seconds_target * per_core / (w.batch * w.seqlen))))
    sl = lambda a: np.ascontiguousarray(gen.to_f64(a[:, :, :nd], io))
    x, dl, z = sl(inp["x"]), sl(inp["delta"]), sl(inp["z"])
    B, C = gen.to_f64(inp["B"], io), gen.to_f64(inp["C"], io)
    h0 = None if inp["h0"] is None else inp["h0"][:, :nd]
    t0 = time.perf_counter()
    oracle.selective_scan(x, dl, inp["A"][:nd], B, C, D=inp["D"][:nd], z=z,
                          delta_bias=inp["delta_bias"][:nd], h0=h0, threads=threads)
    dt = time.perf_counter() - t0
    elems = w.batch * w.seqlen * nd
    return {"value": elems / dt, "unit": "elements/s", "cores": threads, "kind": "oracle",
            "sample": f"all {w.batch} batches x {w.seqlen} steps x first {nd} of {w.d_inner} channels "
                      f"({elems} elements, d_state {w.d_state}), fp64, {dt:.2f} s wall"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=3)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the selective scan here runs on a single MI355X "
              "and has no multi-GPU path (sharding is described in DESIGN.md); use --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from selective_scan_ssm_amd import _lib, ops
    from selective_scan_ssm_amd import inputs as gen

    _lib.load()
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    dev = torch.device("cuda:0")
    w = gen.WORKLOADS[args.workload]
    if w.kind != "scan":
        raise SystemExit("the bench step is the forward scan; pick workload 0, 2 or 3")
    log(f"[bench] generating workload {args.workload} ({w.name})")
    inp = gen.workload_inputs(args.workload)

    def up(a, io):
        if a is None:
            return None
        if io == gen.BF16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    io = inp["io"]
    t = {k: up(inp[k], io) for k in ("x", "delta", "z", "B", "C")}
    t.update({k: up(inp[k], gen.F32) for k in ("A", "D", "delta_bias", "h0")})
    y = torch.empty_like(t["x"])
    last = torch.empty((w.batch, w.d_inner, w.d_state), dtype=torch.float32, device=dev)
    need = _lib.load().ssm_scan_workspace_bytes(w.batch, w.seqlen, w.d_inner, w.d_state,
                                                 _lib.SSM_BF16 if io == gen.BF16 else _lib.SSM_F32)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)

    def step():
        ops.scan_fwd(t["x"], t["delta"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"],
                     delta_bias=t["delta_bias"], h0=t["h0"], return_last_state=True, out=y,
                     last_state_out=last, workspace=ws)

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)   # the stream ops launch on
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s, e in ev:
        s.record(stream)
        step()
        e.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    launch_ms = [s.elapsed_time(e) for s, e in ev]
    ms_per_step = wall * 1e3 / args.steps
    kern_ms = float(np.mean(launch_ms))

    elems = w.batch * w.seqlen * w.d_inner
    io_bytes = 2 if io == gen.BF16 else 4
    alg = algorithmic_bytes(w, io_bytes)
    achieved = alg / (kern_ms * 1e-3) / 1e9
    traffic = traffic_from_profile(SCAN_SOURCES, f"scan_fwd_w{args.workload}")
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
            "kernel": "ssm_scan_fwd (bf16->fp32 B/C widen + scan)",
            "launch_ms_mean": round(kern_ms, 4), "launch_ms_min": round(min(launch_ms), 4),
            "algorithmic_bytes_per_launch": alg}

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle on a sample)")
        cpu = cpu_baseline(inp, w, args.cpu_seconds)

    rec = {"metric": "selective-scan fwd elements/s (B*T*D) and achieved HBM GB/s as % of peak",
           "value": elems / (ms_per_step * 1e-3), "unit": "elements/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "bf16" if io == gen.BF16 else "f32", "data": "synthetic",
           "config": {"workload": w.name, "batch": w.batch, "seqlen": w.seqlen,
                      "d_inner": w.d_inner, "d_state": w.d_state, "io": io,
                      "state": "fp32", "seed": args.workload},
           "roofline": roof, "cpu_baseline": cpu}
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
