#!/usr/bin/env python3
"""Benchmark of the gfx950 selective-scan kernels on one GPU.

Default step: one forward selective scan (ssm_scan_fwd: Delta discretisation,
scan, readout, D skip, SiLU gate, last_state) over a mamba-2.8b-shaped layer:
batch 4, seqlen 8192, d_inner 5120, d_state 16, bf16 x/delta/z/B/C, fp32
A/D/bias/state.  Inputs are seeded synthetic tensors already resident in HBM.
Other workloads (--workload): 0 tiny fp32, 1 SM1 (d_state 1) fp32 through
sm1_scan_fwd, 2 mamba-130m-shaped layer, 4 decode (ssm_state_update over 64
independent layer states, one launch per layer).

Prints one JSON line:  value = elements (B*T*D; decode B*D per layer) per
second over the timed steps, the roofline of the dominant kernel (timed with
HIP events on the stream it is launched on) and the fp64 CPU oracle timed on a
bounded sample of the same workload.

    python bench.py [--steps K] [--warmup W] [--workload 0..4]

--backward times ssm_scan_bwd (the gradient of the scan; workloads 1, 2, 3)
instead, one call per step, against the backward's own VALU roofline; --conv
times the block's causal conv1d + SiLU (ssm_causal_conv1d_fwd, width 4) over
the workload's x against the HBM roofline; --dt-proj times the projection to
delta (ssm_dt_proj, MFMA) of the workload's layer against the HBM roofline,
its output write being the bound; --ssd [NAME] times the Mamba-2
multi-head scan (ssd_scan_fwd) on a Mamba2Block-shaped layer (default
mamba2-2.7b-ssd-layer-bf16) against the HBM roofline.

Profiling helpers (no GPU work of their own beyond what they state):
    python bench.py --copy-calibration       1 GiB device copy, for the
                                             FETCH_SIZE / WRITE_SIZE scale
    python bench.py --summarize-stats DIR    rocprofv3 kernel_stats.csv -> text
    python bench.py --summarize-traffic ...  two --pmc runs + copy runs -> text
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0                       # MI355X HBM3E
# fp32 VALU issue rate of the chip, in fma lane-operations: MI355X's published
# fp32 vector peak 157.3 TFLOP/s is 78.6 T fma/s = 256 CUs x 4 SIMDs x 32
# lanes x 2.4 GHz.  Plain (not packed) fp32 fma issues at that width on gfx950:
# `bench.py --microbench` measures 58.9 T/s at 8 waves per SIMD (the rest is
# the clock under load), 47.8 T/s at 2 and 26.2 T/s at 1.
VALU_PEAK_TSLOTS = 256 * 4 * 32 * 2.4e9 / 1e12
# Transcendentals in fma slots, as measured by the same microbenchmark (issue
# rate of fma over that of the op, 8 waves per SIMD): v_exp_f32 3.1, v_log_f32
# and v_rcp_f32 4.6.
EXP2, LOG2, RCP = 3.1, 4.6, 4.6
# Minimal fp32 VALU slots of the fast (bf16 io) arithmetic:
#  per (t, d, n) item: Delta*A mul, exp2, Delta*x*B mul, decay*h + u fma,
#  C*h fma  -> 4 + EXP2
#  per (t, d) element: 3 widening converts, softplus (add bias, scale, exp2,
#  add, log2, max, fma), Delta*x, SiLU (scale, exp2, add, rcp, mul), D*x fma,
#  gate mul, rounding convert
SLOTS_PER_ITEM = 4 + EXP2
SLOTS_PER_ELEM = 3 + (5 + EXP2 + LOG2) + 1 + (3 + EXP2 + RCP) + 3
# Minimal fp32 VALU slots of the backward (ssm_scan_bwd, bf16 io):
#  per (t, d, n) item: the state again (Delta*A mul, exp2, Delta*x*B mul,
#  decay*h + u fma, C*h fma for the gate's derivative), then the adjoint:
#  g += dy C, a h_{t-1}, g (a h_{t-1}), its A term of dL/dDelta, its Delta
#  term of dA, g B into the per-step sum, g Delta x for dB, dy h for dC,
#  g *= a (9), and one add each for the channel sums of dB and dC
#  per (t, d) element: 4 widening converts, softplus, Delta*x, SiLU and its
#  derivative (scale, exp2, add, rcp, z*s, dy mul, (1 - s), z(1-s)+1, dz
#  product (2)), sigmoid of the softplus input (scale, exp2, add, rcp),
#  dL/dDelta (fma, mul), dx (2), D*x for the readout, dD and dbias sums (2),
#  3 rounding converts
BWD_SLOTS_PER_ITEM = (4 + EXP2) + 9 + 2
BWD_SLOTS_PER_ELEM = 4 + (5 + EXP2 + LOG2) + 1 + (8 + EXP2 + RCP) + (2 + EXP2 + RCP) + 2 + 2 + 1 + 2 + 3
# The block's prologue fused into the scan (ssm_conv_scan_fwd), per element:
# three more widened rows, four taps (fma), SiLU (scale, exp2, add, rcp, mul).
CONV_SLOTS_PER_ELEM = 3 + 4 + (3 + EXP2 + RCP)
COPY_CAL_BYTES = 1 << 30

SOURCES = {
    "scan": ["selective_scan_ssm_amd/csrc/scan_fwd_kernels.h", "selective_scan_ssm_amd/csrc/ssm_device.h"],
    "rows": ["selective_scan_ssm_amd/csrc/scan_fwd_kernels.h", "selective_scan_ssm_amd/csrc/ssm_device.h"],
    "sm1": ["selective_scan_ssm_amd/csrc/sm1_scan.hip", "selective_scan_ssm_amd/csrc/ssm_device.h"],
    "decode": ["selective_scan_ssm_amd/csrc/state_update.hip", "selective_scan_ssm_amd/csrc/ssm_device.h"],
    "conv": ["selective_scan_ssm_amd/csrc/conv1d.hip", "selective_scan_ssm_amd/csrc/ssm_device.h"],
    "ssd": ["selective_scan_ssm_amd/csrc/ssd_scan.hip", "selective_scan_ssm_amd/csrc/ssm_device.h"],
    "ssdline": ["selective_scan_ssm_amd/csrc/ssd_scan.hip", "selective_scan_ssm_amd/csrc/ssm_device.h"],
    "dtproj": ["selective_scan_ssm_amd/csrc/dt_proj.hip", "selective_scan_ssm_amd/csrc/ssm_device.h"],
    "dtprojrows": ["selective_scan_ssm_amd/csrc/dt_proj.hip", "selective_scan_ssm_amd/csrc/ssm_device.h"],
}
# the forward scan runs scan_rows_kernel at d_state 16 and scan_fwd_kernel otherwise
KERNEL_PREFIX = {"scan": "scan_fwd_kernel", "rows": "scan_rows_kernel", "sm1": "sm1_scan_kernel",
                 "decode": "state_update_rows_kernel", "conv": "conv1d_kernel", "ssd": "ssd_chunk_kernel",
                 "ssdline": "ssd_line_kernel", "dtproj": "dt_proj_kernel", "dtprojrows": "dt_proj_rows_kernel"}
# kinds whose one launch runs several kernels: (a pattern every kernel of the
# launch matches, a pattern of the kernel that ends each launch); the others
# run their one kernel per launch
LAUNCH_KERNELS = {
    # the state pass and the carry (time segments only), then the output pass
    "ssdline": (r"ssd_line_kernel<|ssd_carry_kernel<", r"ssd_line_kernel<\d+, \w+, 0>"),
}


def dtproj_kind(w):
    """The kernel ssm_dt_proj runs on a workload's layer: the persistent
    W-resident kernel for bf16 io and dt_rank <= 160, the tiled one otherwise."""
    from selective_scan_ssm_amd import inputs as gen
    _, rank, _, _ = dtproj_shape(w)
    return "dtprojrows" if (w.io == gen.BF16 and rank <= 160) else "dtproj"


def ssd_kind(w):
    """The kernel ssd_scan_fwd runs on an SSD workload: the whole-line kernel
    for bf16 io, head sizes that are multiples of 64 and d_state up to 64,
    the chunk kernel otherwise."""
    from selective_scan_ssm_amd import inputs as gen
    return "ssdline" if (w.io == gen.BF16 and w.headdim % 64 == 0 and w.d_state <= 64) else "ssd"


def grid_of(spec, seqlen):
    """(height, width) of the patch grid the 2-D leg scans: 'HxW', or one row."""
    if spec is None:
        return 1, seqlen
    gh, gw = (int(v) for v in spec.lower().split("x"))
    if gh * gw != seqlen:
        raise SystemExit(f"--grid {spec}: {gh} x {gw} != the workload's {seqlen} steps")
    return gh, gw


def order_visit(direction, spec, seqlen):
    """How the row kernel visits a 2-D order in place at d_state 16 (orders 2
    and 3 of a one-row or one-column grid are orders 0 and 1)."""
    gh, gw = grid_of(spec, seqlen)
    d = direction - 2 if direction >= 2 and (gh == 1 or gw == 1) else direction
    return ["the sequence as stored", "reading each segment from its end",
            "computing each step's patch row, column-major",
            "computing each step's patch row, column-major from the end"][d]


def kind_of(w):
    if w.kind == "scan":
        return "rows" if w.d_state == 16 else "scan"
    return w.kind


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_bytes(w, io_bytes):
    """Bytes the method must move once per launch: x, delta, z read and y
    written per element; B, C per (b, t, n); A, D, delta_bias per channel;
    h0 read (if given) and last_state written.  Decode: the state is read and
    written in place; T = 1."""
    Bt, T, Dd, N = w.batch, w.seqlen, w.d_inner, w.d_state
    b = 4 * Bt * T * Dd * io_bytes
    b += 2 * Bt * T * N * io_bytes
    b += (Dd * N + 2 * Dd) * 4
    if w.h0_kind != "none":
        b += Bt * Dd * N * 4
    b += Bt * Dd * N * 4
    return b


def bwd_algorithmic_bytes(w, io_bytes):
    """Bytes the backward must move once: x, delta, z, dL/dy read and dx,
    ddelta, dz written per element; B, C read and dB, dC written per (b, t, n);
    A, D, bias read and dA, dD, dbias written; h0 read and dh0 written."""
    Bt, T, Dd, N = w.batch, w.seqlen, w.d_inner, w.d_state
    b = 7 * Bt * T * Dd * io_bytes
    b += 4 * Bt * T * N * io_bytes
    b += 2 * (Dd * N + 2 * Dd) * 4
    if w.h0_kind != "none":
        b += Bt * Dd * N * 4
    b += Bt * Dd * N * 4
    return b


def bwd_valu_slots(w):
    items = w.batch * w.seqlen * w.d_inner * w.d_state
    return items * BWD_SLOTS_PER_ITEM + w.batch * w.seqlen * w.d_inner * BWD_SLOTS_PER_ELEM


def valu_slots(w):
    items = w.batch * w.seqlen * w.d_inner * w.d_state
    return items * SLOTS_PER_ITEM + w.batch * w.seqlen * w.d_inner * SLOTS_PER_ELEM


def source_hash(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_file(kind, wname):
    return os.path.join(ROOT, "profiles", f"{KERNEL_PREFIX[kind]}_{wname}_traffic.txt")


def read_kv(path):
    out = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                out[k.strip()] = v.strip()
    return out


def traffic_from_profile(kind, wname):
    """HBM bytes per launch measured by rocprofv3 (FETCH_SIZE + WRITE_SIZE,
    each scaled by the copy-kernel factor), if the stored measurement was taken
    on the current kernel source; else None."""
    path = traffic_file(kind, wname)
    if not os.path.exists(path):
        return None
    rec = read_kv(path)
    if rec.get("source_hash") != source_hash(SOURCES[kind]):
        return None
    return int(float(rec["bytes_per_launch"]))


def host_record():
    """The host the oracle runs on: CPU model, logical CPUs, the CPUs this
    process may use (affinity, and the cgroup's CPU quota where one is set)
    and the ROCm version.  No child process is started."""
    rec = {"cpu_model": "", "logical_cpus": os.cpu_count() or 0}
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    rec["cpu_model"] = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    granted = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    rec["affinity_cpus"] = granted
    try:
        with open("/sys/fs/cgroup/cpu.max") as f:
            quota, period = f.read().split()[:2]
        if quota != "max":
            rec["cgroup_cpu_quota"] = round(int(quota) / int(period), 2)
            granted = min(granted, max(1, int(int(quota) // int(period))))
    except (OSError, ValueError):
        pass
    rec["cpus_granted"] = granted
    for path in ("/opt/rocm/.info/version", "/opt/rocm/.info/version-dev"):
        try:
            with open(path) as f:
                rec["rocm"] = f.read().strip()
            break
        except OSError:
            continue
    return rec


# The oracle's threads: every CPU this process is granted, at most 16 -- the
# CPU share one GPU's job has on the GPU hosts this runs on, whatever the
# machine's own core count.
ORACLE_THREAD_CAP = 16


def oracle_threads():
    return max(1, min(ORACLE_THREAD_CAP, host_record()["cpus_granted"]))


def cpu_baseline(inp, w, seconds_target):
    """The fp64 oracle on a bounded sample of the workload: all batches over
    the full sequence and the first `nd` channels (decode: one layer)."""
    import numpy as np
    import oracle
    from selective_scan_ssm_amd import inputs as gen
    io = inp["io"]
    threads = oracle_threads()
    # about 7e6 elements/s per core at d_state 16: size the sample to about
    # `seconds_target` core-seconds
    per_core = 7e6 * 16 / max(1, w.d_state)
    nd = int(min(w.d_inner, max(64, seconds_target * per_core / (w.batch * w.seqlen))))
    sl = lambda a: None if a is None else np.ascontiguousarray(gen.to_f64(a[:, :, :nd], io))
    x, dl, z = sl(inp["x"]), sl(inp["delta"]), sl(inp["z"])
    B, C = gen.to_f64(inp["B"], io), gen.to_f64(inp["C"], io)
    h0 = None if inp["h0"] is None else np.ascontiguousarray(inp["h0"][:, :nd])
    bias = None if inp["delta_bias"] is None else inp["delta_bias"][:nd]
    D = None if inp["D"] is None else inp["D"][:nd]
    t0 = time.perf_counter()
    oracle.selective_scan(x, dl, np.ascontiguousarray(inp["A"][:nd]), B, C, D=D, z=z,
                          delta_bias=bias, h0=h0, threads=threads)
    dt = time.perf_counter() - t0
    elems = w.batch * w.seqlen * nd
    # the same oracle on one thread, over the first nd1 of those channels
    nd1 = max(1, nd // threads)
    t1 = time.perf_counter()
    oracle.selective_scan(np.ascontiguousarray(x[:, :, :nd1]), np.ascontiguousarray(dl[:, :, :nd1]),
                          np.ascontiguousarray(inp["A"][:nd1]), B, C, D=None if D is None else D[:nd1],
                          z=None if z is None else np.ascontiguousarray(z[:, :, :nd1]),
                          delta_bias=None if bias is None else bias[:nd1],
                          h0=None if h0 is None else np.ascontiguousarray(h0[:, :nd1]), threads=1)
    dt1 = time.perf_counter() - t1
    return {"value": elems / dt, "unit": "elements/s", "cores": threads, "kind": "oracle",
            "value_1_thread": w.batch * w.seqlen * nd1 / dt1,
            "sample": f"all {w.batch} batches x {w.seqlen} steps x first {nd} of {w.d_inner} channels "
                      f"({elems} elements, d_state {w.d_state}), fp64, {dt:.2f} s wall; one thread: "
                      f"first {nd1} channels, {dt1:.2f} s"}


def upload(a, io, dev):
    import numpy as np
    import torch
    from selective_scan_ssm_amd import inputs as gen
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if io == gen.BF16 and a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def device_set(inp, dev, decode=False, sm1=False):
    """One device-resident input/output set (decode: T axis dropped; SM1: N axis dropped)."""
    import torch
    from selective_scan_ssm_amd import inputs as gen
    io = inp["io"]
    t = {}
    for k in ("x", "delta", "z"):
        a = inp[k]
        if a is not None and decode:
            a = a[:, 0, :]
        t[k] = upload(a, io, dev)
    for k in ("B", "C"):
        a = inp[k]
        if decode:
            a = a[:, 0, :]
        elif sm1:
            a = a[:, :, 0]
        t[k] = upload(a, io, dev)
    for k in ("A", "D", "delta_bias", "h0"):
        a = inp[k]
        if a is not None and sm1 and k in ("A", "h0"):
            a = a[..., 0]
        t[k] = upload(a, gen.F32, dev)
    t["y"] = torch.empty_like(t["x"])
    return t


def bench_workload(args, dev):
    import numpy as np
    import torch
    from selective_scan_ssm_amd import _lib, ops
    from selective_scan_ssm_amd import inputs as gen

    lib = _lib.load()
    w = gen.WORKLOADS[args.workload]
    kind = kind_of(w)
    io = w.io
    io_code = _lib.SSM_BF16 if io == gen.BF16 else _lib.SSM_F32
    log(f"[bench] workload {args.workload} ({w.name}): generating inputs")
    inp0 = gen.workload_inputs(args.workload)
    stream = torch.cuda.current_stream(dev)      # the stream ops.* launch on

    if kind == "decode":
        sets = [device_set(inp0, dev, decode=True)]
        for layer in range(1, w.layers):
            sets.append(device_set(gen.workload_inputs(args.workload, layer=layer), dev, decode=True))
        # the state is updated in place: keep it in the set
        for s in sets:
            s["state"] = s["h0"]
        launches = w.layers

        # validate every layer's tensors once through the wrapper, then queue the
        # 64 launches straight through the C ABI so host overhead stays below a
        # launch's duration
        for s in sets:
            ops.state_update(s["state"], s["x"], s["delta"], s["A"], s["B"], s["C"], D=s["D"],
                             z=s["z"], delta_bias=s["delta_bias"], out=s["y"])
        sid = stream.cuda_stream
        p = lambda t: None if t is None else t.data_ptr()
        calls = [(p(s["state"]), p(s["x"]), p(s["delta"]), p(s["delta_bias"]), 1, p(s["A"]), p(s["B"]),
                  p(s["C"]), p(s["D"]), p(s["z"]), p(s["y"]), w.batch, w.d_inner, w.d_state, io_code, sid)
                 for s in sets]
        fn = lib.ssm_state_update

        def step():
            for c in calls:
                rc = fn(*c)
                if rc:
                    raise RuntimeError(lib.ssm_status_string(rc).decode())
    else:
        # rotate input sets until their footprint exceeds the 256 MB last-level
        # cache, so no launch reads inputs a previous launch left cached
        io_b = 2 if io == gen.BF16 else 4
        foot = algorithmic_bytes(w, io_b)
        nset = max(1, math.ceil(600e6 / foot)) if args.rotate is None else args.rotate
        sets = [device_set(inp0, dev, sm1=(kind == "sm1")) for _ in range(nset)]
        N = w.d_state
        for s in sets:
            shape = (w.batch, w.d_inner) if kind == "sm1" else (w.batch, w.d_inner, N)
            s["last"] = torch.empty(shape, dtype=torch.float32, device=dev)
        if kind == "sm1":
            need = lib.sm1_scan_workspace_bytes(w.batch, w.seqlen, w.d_inner, io_code)
        else:
            need = lib.ssm_scan_workspace_bytes(w.batch, w.seqlen, w.d_inner, N, io_code)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
        launches = 1
        cur = [0]

        if args.direction is not None:
            if kind == "sm1":
                raise SystemExit("--direction runs ssm_scan_fwd_2d: use workload 2 or 3")
            gh, gw = grid_of(args.grid, w.seqlen)
            need = lib.ssm_scan_2d_workspace_bytes(w.batch, gh, gw, w.d_inner, N, args.direction, 1, io_code)
            ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)

        def step():
            s = sets[cur[0] % len(sets)]
            cur[0] += 1
            if args.direction is not None:      # the sequence as a patch grid (default: one row)
                ops.scan_fwd_2d(s["x"], s["delta"], s["A"], s["B"], s["C"], gh, gw, args.direction,
                                D=s["D"], z=s["z"], delta_bias=s["delta_bias"], h0=s["h0"],
                                out=s["y"], workspace=ws)
                return
            fn = ops.sm1_scan_fwd if kind == "sm1" else ops.scan_fwd
            fn(s["x"], s["delta"], s["A"], s["B"], s["C"], D=s["D"], z=s["z"],
               delta_bias=s["delta_bias"], h0=s["h0"], return_last_state=True, out=s["y"],
               last_state_out=s["last"], workspace=ws)

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
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
    step_ms = [s.elapsed_time(e) for s, e in ev]
    ms_per_step = wall * 1e3 / args.steps
    launch_ms = float(np.mean(step_ms)) / launches     # mean launch duration, events on `stream`

    elems = w.batch * w.seqlen * w.d_inner * launches
    io_b = 2 if io == gen.BF16 else 4
    alg = algorithmic_bytes(w, io_b)
    hbm_gbs = alg / (launch_ms * 1e-3) / 1e9
    traffic = traffic_from_profile(kind, w.name) if args.direction is None else None
    kname = {"scan": "ssm_scan_fwd (scan_fwd_kernel)",
             "rows": "ssm_scan_fwd (scan_rows_kernel)" if args.direction is None else
                     "ssm_scan_fwd_2d (scan_rows_kernel, " + order_visit(args.direction, args.grid, w.seqlen) + ")",
             "sm1": "sm1_scan_fwd (sm1_scan_kernel)",
             "decode": "ssm_state_update (state_update_rows_kernel)"}[kind]
    if kind in ("scan", "rows") and w.d_state > 1:
        slots = valu_slots(w)
        ach = slots / (launch_ms * 1e-3) / 1e12
        roof = {"bound": "alu", "achieved": round(ach, 3), "peak": round(VALU_PEAK_TSLOTS, 3),
                "unit": "T fp32 fma-equivalent lane-slots/s", "frac": round(ach / VALU_PEAK_TSLOTS, 4),
                "traffic": traffic, "kernel": kname,
                "algorithmic_slots_per_launch": slots,
                "hbm_achieved_GBs": round(hbm_gbs, 1), "hbm_peak_GBs": HBM_PEAK_GBS,
                "hbm_frac": round(hbm_gbs / HBM_PEAK_GBS, 4)}
    else:
        roof = {"bound": "hbm", "achieved": round(hbm_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(hbm_gbs / HBM_PEAK_GBS, 4), "traffic": traffic, "kernel": kname}
    roof.update({"launch_ms_mean": round(launch_ms, 5),
                 "launch_ms_min": round(min(step_ms) / launches, 5),
                 "launch_ms_median": round(float(np.median(step_ms)) / launches, 5),
                 "launch_ms_max": round(max(step_ms) / launches, 5),
                 "algorithmic_bytes_per_launch": alg})

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle on a sample)")
        cpu = cpu_baseline(inp0, w, args.cpu_seconds)

    cfg = {"workload": w.name + ("" if args.direction is None else
                                 f"-order{args.direction}-grid{'x'.join(map(str, grid_of(args.grid, w.seqlen)))}"),
           "batch": w.batch, "seqlen": w.seqlen, "d_inner": w.d_inner,
           "d_state": w.d_state, "io": io, "state": "fp32", "seed": args.workload}
    if kind == "decode":
        cfg["layers"] = w.layers
    elif len(sets) > 1:
        cfg["rotated_input_sets"] = len(sets)
    return {"metric": "selective-scan fwd elements/s (B\u00b7T\u00b7D) and achieved HBM GB/s as % of peak",
            "value": elems / (ms_per_step * 1e-3), "unit": "elements/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "bf16" if io == gen.BF16 else "f32", "data": "synthetic",
            "config": cfg, "roofline": roof, "cpu_baseline": cpu}


def cpu_baseline_bwd(inp, dout, w, seconds_target):
    """The fp64 oracle gradient on a bounded sample: all batches over the full
    sequence and the first `nd` channels."""
    import numpy as np
    import oracle
    from selective_scan_ssm_amd import inputs as gen
    io = inp["io"]
    threads = oracle_threads()
    per_core = 2.5e6 * 16 / max(1, w.d_state)         # the forward's rate / ~3
    nd = int(min(w.d_inner, max(64, seconds_target * per_core / (w.batch * w.seqlen))))
    sl = lambda a: None if a is None else np.ascontiguousarray(gen.to_f64(a[:, :, :nd], io))
    x, dl, z, go = sl(inp["x"]), sl(inp["delta"]), sl(inp["z"]), sl(dout)
    B, C = gen.to_f64(inp["B"], io), gen.to_f64(inp["C"], io)
    h0 = None if inp["h0"] is None else np.ascontiguousarray(inp["h0"][:, :nd])
    bias = None if inp["delta_bias"] is None else inp["delta_bias"][:nd]
    D = None if inp["D"] is None else inp["D"][:nd]
    t0 = time.perf_counter()
    oracle.selective_scan_bwd(x, dl, np.ascontiguousarray(inp["A"][:nd]), B, C, go, D=D, z=z,
                              delta_bias=bias, h0=h0, threads=threads)
    dt = time.perf_counter() - t0
    elems = w.batch * w.seqlen * nd
    return {"value": elems / dt, "unit": "elements/s", "cores": threads, "kind": "oracle",
            "sample": f"gradient, all {w.batch} batches x {w.seqlen} steps x first {nd} of {w.d_inner} "
                      f"channels ({elems} elements, d_state {w.d_state}), fp64, {dt:.2f} s wall"}


def bench_backward(args, dev):
    """ssm_scan_bwd (the gradient of the scan) on a scan workload: one step =
    one backward call with dL/dy resident in HBM."""
    import numpy as np
    import torch
    from selective_scan_ssm_amd import _lib, ops
    from selective_scan_ssm_amd import inputs as gen
    lib = _lib.load()
    w = gen.WORKLOADS[args.workload]
    if w.kind not in ("scan", "sm1"):
        raise SystemExit("--backward needs a scan workload (1, 2 or 3)")
    io = w.io
    io_code = _lib.SSM_BF16 if io == gen.BF16 else _lib.SSM_F32
    log(f"[bench] backward, workload {args.workload} ({w.name}): generating inputs")
    inp = gen.workload_inputs(args.workload)
    rng = np.random.default_rng(1000 + args.workload)
    dout = rng.standard_normal(inp["x"].shape).astype(np.float32)
    if io == gen.BF16:
        dout = gen.bf16_from_f32(dout)
    stream = torch.cuda.current_stream(dev)
    io_b = 2 if io == gen.BF16 else 4
    alg = bwd_algorithmic_bytes(w, io_b)
    nset = max(1, math.ceil(600e6 / alg)) if args.rotate is None else args.rotate
    sets = []
    for _ in range(nset):
        t = device_set(inp, dev)
        t["dout"] = upload(dout, io, dev)
        sets.append(t)
    N = w.d_state
    need = lib.ssm_scan_bwd_workspace_bytes(w.batch, w.seqlen, w.d_inner, N, io_code)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    cur = [0]

    def step():
        s = sets[cur[0] % len(sets)]
        cur[0] += 1
        ops.scan_bwd(s["x"], s["delta"], s["A"], s["B"], s["C"], s["dout"], D=s["D"], z=s["z"],
                     delta_bias=s["delta_bias"], h0=s["h0"], workspace=ws)

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    log(f"[bench] timing {args.steps} steps")
    t0 = time.perf_counter()
    for s, e in ev:
        s.record(stream)
        step()
        e.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = [s.elapsed_time(e) for s, e in ev]
    ms_per_step = wall * 1e3 / args.steps
    call_ms = float(np.mean(step_ms))
    elems = w.batch * w.seqlen * w.d_inner
    slots = bwd_valu_slots(w)
    ach = slots / (call_ms * 1e-3) / 1e12
    hbm = alg / (call_ms * 1e-3) / 1e9
    kname = "ssm_scan_bwd (checkpoint pass + bwd_kernel + bwd_reduce_kernel, timed as one call)"
    if N > 1:       # d_state 16: the per-item work bounds it, as in the forward
        roof = {"bound": "alu", "achieved": round(ach, 3), "peak": round(VALU_PEAK_TSLOTS, 3),
                "unit": "T fp32 fma-equivalent lane-slots/s", "frac": round(ach / VALU_PEAK_TSLOTS, 4),
                "traffic": None, "kernel": kname, "algorithmic_slots_per_launch": slots,
                "hbm_achieved_GBs": round(hbm, 1), "hbm_peak_GBs": HBM_PEAK_GBS,
                "hbm_frac": round(hbm / HBM_PEAK_GBS, 4)}
    else:           # d_state 1: bytes bound it, as in the SM1 forward
        roof = {"bound": "hbm", "achieved": round(hbm, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(hbm / HBM_PEAK_GBS, 4), "traffic": None, "kernel": kname}
    roof.update({"launch_ms_mean": round(call_ms, 5), "launch_ms_min": round(min(step_ms), 5),
                 "launch_ms_median": round(float(np.median(step_ms)), 5), "launch_ms_max": round(max(step_ms), 5),
                 "algorithmic_bytes_per_launch": alg})
    # A training step's alternative: the forward records the checkpoints
    # (ssm_scan_fwd_ckpt) and the backward reuses them (ssm_scan_bwd_ckpt),
    # against the plain forward and the self-contained backward timed above.
    log("[bench] forward with checkpoints and the backward that reuses them")
    fws_need = lib.ssm_scan_workspace_bytes(w.batch, w.seqlen, w.d_inner, N, io_code)
    fws = torch.empty(max(fws_need, 1), dtype=torch.uint8, device=dev)
    ck = torch.empty(ops.ckpt_shape(w.batch, w.seqlen, w.d_inner, N), dtype=torch.float32, device=dev)
    s0 = sets[0]
    y0 = torch.empty_like(s0["x"])
    fwd_args = (s0["x"], s0["delta"], s0["A"], s0["B"], s0["C"])
    fwd_kw = dict(D=s0["D"], z=s0["z"], delta_bias=s0["delta_bias"], h0=s0["h0"], out=y0, workspace=fws)

    def timed(fn, reps=5):
        fn()
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a_, b_ in evs:
            a_.record(stream)
            fn()
            b_.record(stream)
        torch.cuda.synchronize()
        return round(float(np.mean([a_.elapsed_time(b_) for a_, b_ in evs])), 5)

    fwd_ms = timed(lambda: ops.scan_fwd(*fwd_args, **fwd_kw))
    fwd_ck_ms = timed(lambda: ops.scan_fwd(*fwd_args, ckpt_out=ck, **fwd_kw))
    bwd_ck_ms = timed(lambda: ops.scan_bwd(*fwd_args, s0["dout"], D=s0["D"], z=s0["z"], delta_bias=s0["delta_bias"],
                                           h0=s0["h0"], workspace=ws, ckpt=ck))
    roof["with_forward_checkpoints"] = {
        "fwd_ms": fwd_ms, "fwd_ckpt_ms": fwd_ck_ms, "bwd_ckpt_ms": bwd_ck_ms,
        "step_ms": round(fwd_ck_ms + bwd_ck_ms, 5), "step_ms_self_contained": round(fwd_ms + call_ms, 5),
        "note": "training step = forward + backward; the self-contained backward reruns the forward for "
                "its checkpoints, the pair ssm_scan_fwd_ckpt / ssm_scan_bwd_ckpt records them once"}
    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle gradient on a sample)")
        cpu = cpu_baseline_bwd(inp, dout, w, args.cpu_seconds)
    cfg = {"workload": w.name + "-backward", "batch": w.batch, "seqlen": w.seqlen,
           "d_inner": w.d_inner, "d_state": N, "io": io, "state": "fp32", "seed": args.workload}
    if len(sets) > 1:
        cfg["rotated_input_sets"] = len(sets)
    return {"metric": "selective-scan bwd elements/s (B*T*D)",
            "value": elems / (ms_per_step * 1e-3), "unit": "elements/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "bf16" if io == gen.BF16 else "f32", "data": "synthetic",
            "config": cfg, "roofline": roof, "cpu_baseline": cpu}


def dtproj_shape(w):
    """dt_proj of a scan workload's layer: rows B*T, rank = d_model / 16 with
    d_model = d_inner / 2 (expand 2), x_proj rows of rank + 2 d_state."""
    rank = max(1, (w.d_inner // 2) // 16)
    return w.batch * w.seqlen, rank, w.d_inner, rank + 2 * w.d_state


def dtproj_algorithmic_bytes(rows, rank, dim, io_b):
    # the rank columns of each x_proj row and W read once, delta written once
    return (rows * rank + dim * rank + rows * dim) * io_b


def bench_dtproj(args, dev):
    """ssm_dt_proj over a scan workload's layer: one step = the projection of
    all (batch x seqlen) x_proj rows to delta (rows x d_inner)."""
    import numpy as np
    import torch
    from selective_scan_ssm_amd import _lib, ops
    from selective_scan_ssm_amd import inputs as gen
    import oracle
    _lib.load()
    w = gen.WORKLOADS[args.workload]
    if w.kind != "scan":
        raise SystemExit("--dt-proj needs a Mamba layer workload (2 or 3)")
    io = w.io
    io_b = 2 if io == gen.BF16 else 4
    rows, rank, dim, ldx = dtproj_shape(w)
    log(f"[bench] dt_proj, workload {args.workload} ({w.name}): rows {rows} rank {rank} d_inner {dim}")
    inp = gen.make_dtproj_inputs(rows, rank, dim, ldx, io=io, seed=args.workload)
    alg = dtproj_algorithmic_bytes(rows, rank, dim, io_b)
    flops = 2 * rows * rank * dim
    nset = max(1, math.ceil(600e6 / alg)) if args.rotate is None else args.rotate
    xds = [upload(inp["x_dbl"], io, dev) for _ in range(nset)]
    Wd = upload(inp["W"], io, dev)
    outs = [torch.empty((rows, dim), dtype=xds[0].dtype, device=dev) for _ in range(nset)]
    stream = torch.cuda.current_stream(dev)
    cur = [0]

    def step():
        i = cur[0] % nset
        cur[0] += 1
        ops.dt_proj(xds[i][:, :rank], Wd, out=outs[i])

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    t0 = time.perf_counter()
    for s, e in ev:
        s.record(stream)
        step()
        e.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = [s.elapsed_time(e) for s, e in ev]
    ms_per_step = wall * 1e3 / args.steps
    call_ms = float(np.mean(step_ms))
    hbm = alg / (call_ms * 1e-3) / 1e9
    name = w.name + "-dt_proj"
    mfma_peak = 2500.0 if io == gen.BF16 else 157.3
    roof = {"bound": "hbm", "achieved": round(hbm, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(hbm / HBM_PEAK_GBS, 4), "traffic": traffic_from_profile(dtproj_kind(w), name),
            "kernel": f"ssm_dt_proj ({KERNEL_PREFIX[dtproj_kind(w)]})",
            "launch_ms_mean": round(call_ms, 5), "launch_ms_min": round(min(step_ms), 5),
            "launch_ms_median": round(float(np.median(step_ms)), 5), "launch_ms_max": round(max(step_ms), 5),
            "algorithmic_bytes_per_launch": alg,
            "mfma": {"achieved": round(flops / (call_ms * 1e-3) / 1e12, 2), "peak": mfma_peak,
                     "unit": "TFLOP/s", "flops_per_launch": flops}}
    cpu = None
    if not args.no_cpu_baseline:
        threads = oracle_threads()
        # about 3e9 multiply-adds per core-second (measured): size the sample to
        # about `cpu_seconds` core-seconds
        nr = int(min(rows, max(64, args.cpu_seconds * 3e9 / (rank * dim))))
        x64 = gen.to_f64(inp["x_dbl"][:nr], io)
        t1 = time.perf_counter()
        oracle.dt_proj(x64, gen.to_f64(inp["W"], io), threads=threads)
        dt = time.perf_counter() - t1
        cpu = {"value": nr * dim / dt, "unit": "elements/s", "cores": threads, "kind": "oracle",
               "sample": f"dt_proj, the first {nr} of {rows} rows, all {dim} channels, rank {rank}, "
                         f"fp64, {dt:.2f} s wall"}
    cfg = {"workload": name, "rows": rows, "rank": rank, "d_inner": dim, "x_proj_row": ldx, "io": io,
           "seed": args.workload}
    if nset > 1:
        cfg["rotated_input_sets"] = nset
    return {"metric": "dt_proj elements/s (rows*d_inner)", "value": rows * dim / (ms_per_step * 1e-3),
            "unit": "elements/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16" if io == gen.BF16 else "f32", "data": "synthetic",
            "config": cfg, "roofline": roof, "cpu_baseline": cpu}


def bench_conv(args, dev):
    """ssm_causal_conv1d_fwd (width 4, SiLU) over the x of a scan workload:
    one step = one convolution of the whole (batch, seqlen, d_inner) tensor."""
    import numpy as np
    import torch
    from selective_scan_ssm_amd import _lib, ops
    from selective_scan_ssm_amd import inputs as gen
    import oracle
    _lib.load()
    w = gen.WORKLOADS[args.workload]
    if w.kind not in ("scan", "sm1"):
        raise SystemExit("--conv needs a scan workload (1, 2 or 3)")
    io, K = w.io, 4
    io_b = 2 if io == gen.BF16 else 4
    log(f"[bench] conv1d, workload {args.workload} ({w.name}): generating inputs")
    inp = gen.workload_inputs(args.workload)
    rng = np.random.default_rng(2000 + args.workload)
    wt = (rng.standard_normal((w.d_inner, K)) * 0.5).astype(np.float32)
    bias = rng.standard_normal(w.d_inner).astype(np.float32)
    alg = 2 * w.batch * w.seqlen * w.d_inner * io_b + w.d_inner * (K + 1) * 4
    nset = max(1, math.ceil(600e6 / alg)) if args.rotate is None else args.rotate
    xs = [upload(inp["x"], io, dev) for _ in range(nset)]
    outs = [torch.empty_like(xs[0]) for _ in range(nset)]
    wd, bd = upload(wt, gen.F32, dev), upload(bias, gen.F32, dev)
    stream = torch.cuda.current_stream(dev)
    cur = [0]

    def step():
        i = cur[0] % nset
        cur[0] += 1
        ops.causal_conv1d(xs[i], wd, bd, silu=True, out=outs[i])

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    t0 = time.perf_counter()
    for s, e in ev:
        s.record(stream)
        step()
        e.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = [s.elapsed_time(e) for s, e in ev]
    ms_per_step = wall * 1e3 / args.steps
    call_ms = float(np.mean(step_ms))
    hbm = alg / (call_ms * 1e-3) / 1e9
    roof = {"bound": "hbm", "achieved": round(hbm, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(hbm / HBM_PEAK_GBS, 4), "traffic": traffic_from_profile("conv", w.name + "-conv1d"),
            "kernel": "ssm_causal_conv1d_fwd (conv1d_kernel)",
            "launch_ms_mean": round(call_ms, 5), "launch_ms_min": round(min(step_ms), 5),
            "launch_ms_median": round(float(np.median(step_ms)), 5), "launch_ms_max": round(max(step_ms), 5),
            "algorithmic_bytes_per_launch": alg}
    cpu = None
    if not args.no_cpu_baseline:
        threads = oracle_threads()
        nd = int(min(w.d_inner, max(64, args.cpu_seconds * 4e7 / (w.batch * w.seqlen))))
        xs64 = np.ascontiguousarray(gen.to_f64(inp["x"][:, :, :nd], io))
        t1 = time.perf_counter()
        oracle.causal_conv1d(xs64, wt[:nd], bias[:nd], None, silu=True, threads=threads)
        dt = time.perf_counter() - t1
        el = w.batch * w.seqlen * nd
        cpu = {"value": el / dt, "unit": "elements/s", "cores": threads, "kind": "oracle",
               "sample": f"conv1d, all {w.batch} batches x {w.seqlen} steps x first {nd} of "
                         f"{w.d_inner} channels ({el} elements, width 4), fp64, {dt:.2f} s wall"}
    elems = w.batch * w.seqlen * w.d_inner
    cfg = {"workload": w.name + "-conv1d", "batch": w.batch, "seqlen": w.seqlen, "d_inner": w.d_inner,
           "width": K, "io": io, "seed": args.workload}
    if nset > 1:
        cfg["rotated_input_sets"] = nset
    return {"metric": "causal conv1d + SiLU elements/s (B*T*D)", "value": elems / (ms_per_step * 1e-3),
            "unit": "elements/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16" if io == gen.BF16 else "f32", "data": "synthetic",
            "config": cfg, "roofline": roof, "cpu_baseline": cpu}


def bench_conv_scan(args, dev):
    """ssm_conv_scan_fwd on a d_state-16 scan workload: the causal conv1d
    (width 4) + SiLU run inside the scan kernel, one launch.  Timed beside
    the same work as two launches (ssm_causal_conv1d_fwd into a buffer, then
    ssm_scan_fwd), with HIP events on the stream both launch on."""
    import numpy as np
    import torch
    from selective_scan_ssm_amd import _lib, ops
    from selective_scan_ssm_amd import inputs as gen
    import oracle
    _lib.load()
    w = gen.WORKLOADS[args.workload]
    if kind_of(w) != "rows":
        raise SystemExit("--conv-scan needs a d_state-16 scan workload (2 or 3)")
    io, K = w.io, 4
    io_b = 2 if io == gen.BF16 else 4
    log(f"[bench] conv1d + scan, workload {args.workload} ({w.name}): generating inputs")
    inp = gen.workload_inputs(args.workload)
    cp = gen.make_conv_params(w.batch, w.d_inner, K, io=io, seed=31)
    alg = algorithmic_bytes(w, io_b) + w.d_inner * (K + 1) * 4
    nset = max(1, math.ceil(600e6 / alg)) if args.rotate is None else args.rotate
    sets = [device_set(inp, dev) for _ in range(nset)]
    wd, bd = upload(cp["conv_w"], gen.F32, dev), upload(cp["conv_b"], gen.F32, dev)
    N = w.d_state
    for st in sets:
        st["last"] = torch.empty((w.batch, w.d_inner, N), dtype=torch.float32, device=dev)
    need = ops.scan_workspace_bytes(w.batch, w.seqlen, w.d_inner, N, sets[0]["x"].dtype)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    xc = torch.empty_like(sets[0]["x"])          # the two-launch path's filtered x
    stream = torch.cuda.current_stream(dev)
    cur = [0]

    def fused():
        st = sets[cur[0] % nset]
        cur[0] += 1
        ops.conv_scan_fwd(st["x"], wd, st["delta"], st["A"], st["B"], st["C"], conv_bias=bd, D=st["D"],
                          z=st["z"], delta_bias=st["delta_bias"], out=st["y"], workspace=ws)

    def two_launches():
        st = sets[cur[0] % nset]
        cur[0] += 1
        ops.causal_conv1d(st["x"], wd, bd, silu=True, out=xc)
        ops.scan_fwd(xc, st["delta"], st["A"], st["B"], st["C"], D=st["D"], z=st["z"],
                     delta_bias=st["delta_bias"], return_last_state=True, out=st["y"],
                     last_state_out=st["last"], workspace=ws)

    def timed(fn, steps, warm):
        for _ in range(warm):
            fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        t0 = time.perf_counter()
        for a, b in ev:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / steps, [a.elapsed_time(b) for a, b in ev]

    log(f"[bench] two launches: warmup {args.warmup}, {args.steps} steps")
    two_ms, two_ev = timed(two_launches, args.steps, args.warmup)
    log(f"[bench] fused: warmup {args.warmup}, {args.steps} steps")
    ms_per_step, step_ms = timed(fused, args.steps, args.warmup)
    call_ms = float(np.mean(step_ms))
    slots = valu_slots(w) + w.batch * w.seqlen * w.d_inner * CONV_SLOTS_PER_ELEM
    ach = slots / (call_ms * 1e-3) / 1e12
    hbm = alg / (call_ms * 1e-3) / 1e9
    roof = {"bound": "alu", "achieved": round(ach, 3), "peak": round(VALU_PEAK_TSLOTS, 3),
            "unit": "T fp32 fma-equivalent lane-slots/s", "frac": round(ach / VALU_PEAK_TSLOTS, 4),
            "traffic": None, "kernel": "ssm_conv_scan_fwd (scan_rows_kernel with the conv prologue)",
            "algorithmic_slots_per_launch": slots, "hbm_achieved_GBs": round(hbm, 1),
            "hbm_peak_GBs": HBM_PEAK_GBS, "hbm_frac": round(hbm / HBM_PEAK_GBS, 4),
            "launch_ms_mean": round(call_ms, 5), "launch_ms_min": round(min(step_ms), 5),
            "launch_ms_median": round(float(np.median(step_ms)), 5), "launch_ms_max": round(max(step_ms), 5),
            "algorithmic_bytes_per_launch": alg,
            "two_launches_ms_mean": round(float(np.mean(two_ev)), 5),
            "two_launches_ms_per_step": round(two_ms, 4)}
    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle conv1d + scan on a sample)")
        threads = oracle_threads()
        nd = int(min(w.d_inner, max(64, args.cpu_seconds * 7e6 / (w.batch * w.seqlen))))
        sl = lambda a: None if a is None else np.ascontiguousarray(gen.to_f64(a[:, :, :nd], io))
        t1 = time.perf_counter()
        xo, _ = oracle.causal_conv1d(sl(inp["x"]), cp["conv_w"][:nd], cp["conv_b"][:nd], None, silu=True,
                                     threads=threads)
        oracle.selective_scan(xo, sl(inp["delta"]), np.ascontiguousarray(inp["A"][:nd]),
                              gen.to_f64(inp["B"], io), gen.to_f64(inp["C"], io), D=inp["D"][:nd],
                              z=sl(inp["z"]), delta_bias=inp["delta_bias"][:nd], threads=threads)
        dt = time.perf_counter() - t1
        el = w.batch * w.seqlen * nd
        cpu = {"value": el / dt, "unit": "elements/s", "cores": threads, "kind": "oracle",
               "sample": f"conv1d + scan, all {w.batch} batches x {w.seqlen} steps x first {nd} of "
                         f"{w.d_inner} channels ({el} elements, width 4, d_state 16), fp64, {dt:.2f} s wall"}
    elems = w.batch * w.seqlen * w.d_inner
    cfg = {"workload": w.name + "-conv-scan", "batch": w.batch, "seqlen": w.seqlen, "d_inner": w.d_inner,
           "d_state": N, "width": K, "io": io, "state": "fp32", "seed": args.workload}
    if nset > 1:
        cfg["rotated_input_sets"] = nset
    return {"metric": "conv1d + SiLU + selective-scan fwd elements/s (B*T*D)",
            "value": elems / (ms_per_step * 1e-3), "unit": "elements/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16" if io == gen.BF16 else "f32",
            "data": "synthetic", "config": cfg, "roofline": roof, "cpu_baseline": cpu}


def ssd_algorithmic_bytes(w, io_bytes):
    """x, z read and y written (B T H P each), dt (B T H), B and C (B T N),
    and the per-head A, D, dt_bias (fp32)."""
    Bt, T, H, P, N = w.batch, w.seqlen, w.n_heads, w.headdim, w.d_state
    return (3 * Bt * T * H * P + Bt * T * H + 2 * Bt * T * N) * io_bytes + 3 * H * 4


def bench_ssd(args, dev):
    """ssd_scan_fwd over a Mamba2Block-shaped layer: one step = one launch
    over the whole (batch, seqlen, heads, head size) input."""
    import numpy as np
    import torch
    from selective_scan_ssm_amd import _lib, ops
    from selective_scan_ssm_amd import inputs as gen
    import oracle
    _lib.load()
    w = gen.SSD_WORKLOADS[args.ssd]
    io = w.io
    io_b = 2 if io == gen.BF16 else 4
    log(f"[bench] ssd scan, {w.name}: generating inputs")
    inp = gen.ssd_workload_inputs(w.name, seed=1)
    alg = ssd_algorithmic_bytes(w, io_b)
    nset = max(1, math.ceil(600e6 / alg)) if args.rotate is None else args.rotate
    sets = []
    for _ in range(nset):
        t = {k: upload(inp[k], io, dev) for k in ("x", "dt", "z", "B", "C")}
        t.update({k: upload(inp[k], gen.F32, dev) for k in ("A", "D", "dt_bias")})
        t["y"] = torch.empty_like(t["x"])
        sets.append(t)
    stream = torch.cuda.current_stream(dev)
    cur = [0]

    def step():
        t = sets[cur[0] % nset]
        cur[0] += 1
        ops.ssd_scan_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"], dt_bias=t["dt_bias"],
                         out=t["y"])

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    t0 = time.perf_counter()
    for s, e in ev:
        s.record(stream)
        step()
        e.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = [s.elapsed_time(e) for s, e in ev]
    ms_per_step = wall * 1e3 / args.steps
    call_ms = float(np.mean(step_ms))
    hbm = alg / (call_ms * 1e-3) / 1e9
    roof = {"bound": "hbm", "achieved": round(hbm, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(hbm / HBM_PEAK_GBS, 4), "traffic": traffic_from_profile(ssd_kind(w), w.name),
            "kernel": f"ssd_scan_fwd ({KERNEL_PREFIX[ssd_kind(w)]})",
            "launch_ms_mean": round(call_ms, 5), "launch_ms_min": round(min(step_ms), 5),
            "launch_ms_median": round(float(np.median(step_ms)), 5), "launch_ms_max": round(max(step_ms), 5),
            "algorithmic_bytes_per_launch": alg}
    cpu = None
    if not args.no_cpu_baseline:
        # the oracle on every batch row and head, the first nc channels of each
        # head (about 5e8 state updates -- one channel, step and n -- per core-second)
        threads = oracle_threads()
        nc = int(min(w.headdim, max(1, args.cpu_seconds * 5e8 / (w.batch * w.seqlen * w.n_heads * w.d_state))))
        f64 = lambda a: np.ascontiguousarray(gen.to_f64(a, io))
        xs = np.ascontiguousarray(f64(inp["x"])[:, :, :, :nc])
        zs = np.ascontiguousarray(f64(inp["z"])[:, :, :, :nc])
        t1 = time.perf_counter()
        oracle.ssd_scan(xs, f64(inp["dt"]), inp["A"], f64(inp["B"]), f64(inp["C"]), D=inp["D"], z=zs,
                        dt_bias=inp["dt_bias"], threads=threads)
        dt = time.perf_counter() - t1
        el = w.batch * w.seqlen * w.n_heads * nc
        cpu = {"value": el / dt, "unit": "elements/s", "cores": threads, "kind": "oracle",
               "sample": f"all {w.batch} batch rows x {w.seqlen} steps x {w.n_heads} heads x first {nc} of "
                         f"{w.headdim} channels ({el} elements, d_state {w.d_state}), fp64, {dt:.2f} s wall"}
    elems = w.batch * w.seqlen * w.n_heads * w.headdim
    cfg = {"workload": w.name, "batch": w.batch, "seqlen": w.seqlen, "d_model": w.d_model,
           "n_heads": w.n_heads, "headdim": w.headdim, "d_state": w.d_state, "chunk": 64, "io": io}
    if nset > 1:
        cfg["rotated_input_sets"] = nset
    return {"metric": "Mamba-2 SSD scan elements/s (B*T*H*P)", "value": elems / (ms_per_step * 1e-3),
            "unit": "elements/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16" if io == gen.BF16 else "f32", "data": "synthetic",
            "config": cfg, "roofline": roof, "cpu_baseline": cpu}


def device_record():
    """Name, CUs and (best effort) the current clocks of GPU 0, the clocks read
    from the amdgpu driver's DPM tables in sysfs (the level marked '*'); no
    child process is started, so the record is safe under a profiler that has
    initialised the GPU before the program runs."""
    import glob
    import torch
    pr = torch.cuda.get_device_properties(0)
    rec = {"name": pr.name, "arch": getattr(pr, "gcnArchName", ""), "cus": pr.multi_processor_count}
    try:
        cards = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        if len(cards) == 1:                           # one GPU: its clocks are unambiguous
            clocks = []
            for table in ("pp_dpm_sclk", "pp_dpm_mclk"):
                with open(cards[0].replace("pp_dpm_sclk", table)) as f:
                    clocks += [f"{table[-4:]} {ln.split(':', 1)[1].replace('*', '').strip()}"
                               for ln in f if ln.rstrip().endswith("*")]
            rec["clocks"] = clocks
    except Exception:                                 # noqa: BLE001 -- the record is optional
        pass
    return rec


def bench_micro(args, dev):
    """Measured ceilings: a 1 GiB 16-byte copy (read + write bandwidth), and
    the issue rate of fp32 fma and of v_exp_f32 over the whole chip."""
    import numpy as np
    import torch
    from selective_scan_ssm_amd import _lib
    lib = _lib.load_bench()
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream

    def timed(fn, reps):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a, b in ev:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in ev]

    nbytes = COPY_CAL_BYTES
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)

    def copy():
        rc = lib.ssm_mb_copy(src.data_ptr(), dst.data_ptr(), nbytes, sh)
        if rc:
            raise RuntimeError(f"ssm_mb_copy failed ({rc})")

    ms = timed(copy, 10)
    copy_gbs = 2 * nbytes / (float(np.median(ms)) * 1e-3) / 1e9
    del src, dst
    iters = 4096
    out = torch.empty(256 * 4 * 8 // 4 * 256, dtype=torch.float32, device=dev)
    rates = {}
    for wps in (1, 2, 8):                              # waves per SIMD over the whole chip
        blocks = 256 * 4 * wps // 4
        for op, name in ((0, "fma"), (1, "exp2"), (2, "log2"), (3, "rcp")):
            if wps != 8 and op != 0:
                continue
            def run(op=op, blocks=blocks):
                rc = lib.ssm_mb_valu(op, out.data_ptr(), blocks, iters, sh)
                if rc:
                    raise RuntimeError(f"ssm_mb_valu failed ({rc})")
            ms = timed(run, 10)
            rates[f"{name}_{wps}w"] = blocks * 256 * iters * 8 / (float(np.median(ms)) * 1e-3) / 1e12
    fma = rates["fma_8w"]
    return {"metric": "measured ceilings", "copy_read_write_GBs": round(copy_gbs, 1),
            "copy_frac_of_8TBs": round(copy_gbs / HBM_PEAK_GBS, 4),
            "valu_T_lane_ops_per_s": {k: round(v, 3) for k, v in rates.items()},
            "valu_peak_T_slots": round(VALU_PEAK_TSLOTS, 3),
            "fma_frac_of_peak": round(fma / VALU_PEAK_TSLOTS, 4),
            "fma_slots_each": {k: round(fma / rates[f"{k}_8w"], 3) for k in ("exp2", "log2", "rcp")},
            "device": device_record(),
            "note": "copy: 1 GiB, 16-byte non-temporal loads and stores; VALU: 256 lanes per workgroup, "
                    "1, 2 or 8 waves per SIMD over 256 CUs, 4096 steps x 8 independent chains per lane"}


def copy_calibration():
    """A plain device copy of COPY_CAL_BYTES, three times: under rocprofv3
    --pmc its FETCH_SIZE / WRITE_SIZE per dispatch give the counter scale."""
    import torch
    dev = torch.device("cuda:0")
    n = COPY_CAL_BYTES // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_CAL_BYTES}), flush=True)


# ---------------------------------------------------------------- summaries

def _rows(d, name):
    paths = glob.glob(os.path.join(d, "**", name), recursive=True)
    if not paths:
        raise SystemExit(f"no {name} under {d}")
    with open(max(paths, key=os.path.getmtime), newline="") as f:   # the latest run in d
        return list(csv.DictReader(f))


def summarize_stats(d, command):
    """Text summary of a rocprofv3 --kernel-trace --stats run (kernel_stats.csv)."""
    rows = _rows(d, "*kernel_stats.csv")
    lines = [f"command: {command}", "", "| kernel | calls | total ms | avg us | min us | max us | % |",
             "|---|---|---|---|---|---|---|"]
    for r in rows:
        name = r["Name"].replace("(anonymous namespace)::", "")
        if name.startswith("void "):
            name = name[5:]
        short = name.split("(")[0][:110]
        lines.append(f"| {short} | {r['Calls']} | {float(r['TotalDurationNs'])/1e6:.3f} | "
                     f"{float(r['AverageNs'])/1e3:.2f} | {float(r['MinNs'])/1e3:.2f} | "
                     f"{float(r['MaxNs'])/1e3:.2f} | {float(r['Percentage']):.2f} |")
    return "\n".join(lines) + "\n"


def _counter_per_launch(d, counter, kind):
    """Median over launches of the counter summed over every kernel of a
    launch (dispatches taken in order, a launch closed by its last kernel),
    and the number of launches."""
    every, last = LAUNCH_KERNELS.get(kind, (re.escape(KERNEL_PREFIX[kind]),) * 2)
    per = {}
    for r in _rows(d, "*counter_collection.csv"):
        if r["Counter_Name"] != counter or not re.search(every, r["Kernel_Name"]):
            continue
        k = int(r["Dispatch_Id"])
        per[k] = (r["Kernel_Name"], per.get(k, ("", 0.0))[1] + float(r["Counter_Value"]))
    launches, acc = [], 0.0
    for k in sorted(per):
        name, v = per[k]
        acc += v
        if re.search(last, name):
            launches.append(acc)
            acc = 0.0
    if not launches:
        raise SystemExit(f"no {counter} rows for {kind} launches in {d}")
    v = sorted(launches)
    return v[len(v) // 2], len(v)


def _counter_per_dispatch(d, counter, kernel_prefix):
    vals = {}
    for r in _rows(d, "*counter_collection.csv"):
        if r["Counter_Name"] != counter:
            continue
        kn = r["Kernel_Name"]
        if kernel_prefix not in kn:
            continue
        key = r["Dispatch_Id"]
        vals[key] = vals.get(key, 0.0) + float(r["Counter_Value"])
    if not vals:
        raise SystemExit(f"no {counter} rows for {kernel_prefix} in {d}")
    v = sorted(vals.values())
    return v[len(v) // 2], len(v)


def summarize_traffic(kind, wname, fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, commands,
                      alg_bytes):
    pre = KERNEL_PREFIX[kind]
    cf, _ = _counter_per_dispatch(copy_fetch_dir, "FETCH_SIZE", "copyBuffer")
    cw, _ = _counter_per_dispatch(copy_write_dir, "WRITE_SIZE", "copyBuffer")
    kib = COPY_CAL_BYTES / 1024
    f_fac, w_fac = kib / cf, kib / cw
    kf, nf = _counter_per_launch(fetch_dir, "FETCH_SIZE", kind)
    kw, nw = _counter_per_launch(write_dir, "WRITE_SIZE", kind)
    fb, wb = kf * f_fac * 1024, kw * w_fac * 1024
    total = fb + wb
    every = LAUNCH_KERNELS.get(kind, (pre,))[0].replace("\\", "").replace("<", "").replace("|", ", ")
    lines = [
        f"# HBM traffic of {pre} on {wname}, from rocprofv3 --pmc (median over launches; "
        f"a launch counts every kernel it runs: {every})",
        *[f"# command: {c}" for c in commands],
        f"kernel: {pre}",
        f"workload: {wname}",
        f"source_hash: {source_hash(SOURCES[kind])}",
        f"copy_calibration_bytes: {COPY_CAL_BYTES}",
        f"copy_FETCH_SIZE_KiB: {cf:.1f}",
        f"copy_WRITE_SIZE_KiB: {cw:.1f}",
        f"fetch_scale: {f_fac:.4f}",
        f"write_scale: {w_fac:.4f}",
        f"kernel_FETCH_SIZE_KiB: {kf:.1f}  (per launch, {nf} launches)",
        f"kernel_WRITE_SIZE_KiB: {kw:.1f}  (per launch, {nw} launches)",
        f"fetch_bytes: {fb:.0f}",
        f"write_bytes: {wb:.0f}",
        f"bytes_per_launch: {total:.0f}",
        f"algorithmic_bytes_per_launch: {alg_bytes}",
        f"traffic_over_algorithmic: {total / alg_bytes:.4f}",
    ]
    return "\n".join(lines) + "\n"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=3)
    ap.add_argument("--rotate", type=int, default=None, help="input sets to rotate (default: enough to exceed 600 MB)")
    ap.add_argument("--cpu-seconds", type=float, default=20.0, help="oracle sample size in core-seconds")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--backward", action="store_true",
                    help="time ssm_scan_bwd (the gradient) on a scan workload instead of the forward")
    ap.add_argument("--grid", default=None, metavar="HxW",
                    help="with --direction: the sequence as an H x W patch grid (default 1 x seqlen)")
    ap.add_argument("--direction", type=int, default=None,
                    help="scan order through ssm_scan_fwd_2d (height 1): 0 forward, 1 reversed")
    ap.add_argument("--conv-scan", action="store_true",
                    help="time ssm_conv_scan_fwd (conv1d + SiLU fused into the d_state-16 scan) on a scan "
                         "workload, beside the two separate launches")
    ap.add_argument("--conv", action="store_true",
                    help="time ssm_causal_conv1d_fwd (width 4, SiLU) on a scan workload's x instead")
    ap.add_argument("--dt-proj", action="store_true",
                    help="time ssm_dt_proj (the projection to delta) of a scan workload's layer instead")
    ap.add_argument("--ssd", nargs="?", const="mamba2-2.7b-ssd-layer-bf16", default=None,
                    help="time ssd_scan_fwd (the Mamba-2 multi-head scan) on the named layer shape instead")
    ap.add_argument("--microbench", action="store_true",
                    help="measure the copy bandwidth and the fp32 fma / v_exp_f32 issue rates instead")
    ap.add_argument("--summarize-stats", nargs=2, metavar=("DIR", "COMMAND"))
    ap.add_argument("--summarize-traffic", nargs=7,
                    metavar=("WORKLOAD", "FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR",
                             "KERNEL_COMMAND", "COPY_COMMAND"))
    args = ap.parse_args()

    if args.summarize_stats:
        sys.stdout.write(summarize_stats(*args.summarize_stats))
        return
    if args.summarize_traffic:
        from selective_scan_ssm_amd import inputs as gen
        wl, fd, wd, cfd, cwd, kcmd, ccmd = args.summarize_traffic
        if wl.startswith("ssd:"):      # "ssd:NAME": the Mamba-2 scan on that layer shape
            w = gen.SSD_WORKLOADS[wl[4:]]
            kind, wname = ssd_kind(w), w.name
            alg = ssd_algorithmic_bytes(w, 2 if w.io == gen.BF16 else 4)
        elif wl.startswith("dtproj"):  # "dtproj3": dt_proj of workload 3's layer
            w = gen.WORKLOADS[int(wl[6:])]
            kind, wname = dtproj_kind(w), w.name + "-dt_proj"
            rows, rank, dim, _ = dtproj_shape(w)
            alg = dtproj_algorithmic_bytes(rows, rank, dim, 2 if w.io == gen.BF16 else 4)
        elif wl.startswith("conv"):    # "conv3": the conv1d over workload 3's x
            w = gen.WORKLOADS[int(wl[4:])]
            kind, wname = "conv", w.name + "-conv1d"
            alg = 2 * w.batch * w.seqlen * w.d_inner * (2 if w.io == gen.BF16 else 4) + w.d_inner * 5 * 4
        else:
            w = gen.WORKLOADS[int(wl)]
            kind, wname = kind_of(w), w.name
            alg = algorithmic_bytes(w, 2 if w.io == gen.BF16 else 4)
        cmds = [kcmd.replace("{COUNTER}", c) for c in ("FETCH_SIZE", "WRITE_SIZE")]
        cmds += [ccmd.replace("{COUNTER}", c) for c in ("FETCH_SIZE", "WRITE_SIZE")]
        text = summarize_traffic(kind, wname, fd, wd, cfd, cwd, cmds, alg)
        with open(traffic_file(kind, wname), "w") as f:
            f.write(text)
        sys.stdout.write(text)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the selective scan here runs on a single MI355X "
              "and has no multi-GPU path; use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    if args.copy_calibration:
        copy_calibration()
        return
    from selective_scan_ssm_amd import _lib
    _lib.load()
    fn = (bench_backward if args.backward else bench_conv if args.conv else
          bench_conv_scan if args.conv_scan else bench_dtproj if args.dt_proj else
          bench_ssd if args.ssd is not None else bench_micro if args.microbench else bench_workload)
    rec = fn(args, torch.device("cuda:0"))
    # the GPU's name, CUs and clocks, read after the timed region
    rec.setdefault("device", device_record())
    if isinstance(rec.get("cpu_baseline"), dict):
        rec["cpu_baseline"]["host"] = host_record()
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
