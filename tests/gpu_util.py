"""Helpers of the GPU parity tests: move seeded inputs to the device, run the
HIP path through the C ABI wrappers, run the fp64 oracle on the same values,
and measure the error the way the tolerances are stated."""
from __future__ import annotations

import os
import sys

import numpy as np

import oracle
from selective_scan_ssm_amd import inputs as gen

IO_KEYS = ("x", "delta", "z", "B", "C")
F32_KEYS = ("A", "D", "delta_bias", "h0")
TOL = {gen.F32: 1e-5, gen.BF16: 2e-2}
ORACLE_THREADS = min(16, os.cpu_count() or 1)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_torch(arr, io, device="cuda"):
    import torch
    if arr is None:
        return None
    if io == gen.BF16 and arr.dtype == np.uint16:
        return torch.from_numpy(arr.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(arr)).to(device)


def from_torch(t):
    import torch
    if t is None:
        return None
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return gen.f32_from_bf16(t.view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


def device_inputs(inp, device="cuda"):
    io = inp["io"]
    out = {k: to_torch(inp[k], io, device) for k in IO_KEYS}
    out.update({k: to_torch(inp[k], gen.F32, device) for k in F32_KEYS})
    return out


def decoded(inp):
    """fp64 copies of the inputs, exactly as the GPU reads them."""
    io = inp["io"]
    d = {k: (None if inp[k] is None else gen.to_f64(inp[k], io)) for k in IO_KEYS}
    d.update({k: (None if inp[k] is None else np.asarray(inp[k], np.float64)) for k in F32_KEYS})
    return d


def run_scan(inp, softplus=True, sm1=False, last=True, device="cuda"):
    import torch
    from selective_scan_ssm_amd import ops
    t = device_inputs(inp, device)
    if sm1:
        r = ops.sm1_scan_fwd(t["x"], t["delta"], t["A"][:, 0].contiguous(), t["B"][..., 0].contiguous(),
                             t["C"][..., 0].contiguous(), D=t["D"], z=t["z"], delta_bias=t["delta_bias"],
                             delta_softplus=softplus,
                             h0=None if t["h0"] is None else t["h0"][..., 0].contiguous(),
                             return_last_state=last)
    else:
        r = ops.scan_fwd(t["x"], t["delta"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"],
                         delta_bias=t["delta_bias"], delta_softplus=softplus, h0=t["h0"],
                         return_last_state=last)
    torch.cuda.synchronize()
    if last:
        y, ls = r
        ls = from_torch(ls)
        if sm1:
            ls = ls[..., None]
        return from_torch(y), ls
    return from_torch(r), None


def run_oracle(inp, softplus=True, d_index=None):
    """Oracle on all chains, or only on channels d_index (all batches)."""
    d = decoded(inp)
    if d_index is not None:
        di = np.asarray(d_index)
        sl = lambda a: None if a is None else np.ascontiguousarray(a[:, :, di])
        d = dict(d, x=sl(d["x"]), delta=sl(d["delta"]), z=sl(d["z"]),
                 A=d["A"][di], D=None if d["D"] is None else d["D"][di],
                 delta_bias=None if d["delta_bias"] is None else d["delta_bias"][di],
                 h0=None if d["h0"] is None else np.ascontiguousarray(d["h0"][:, di]))
    return oracle.selective_scan(d["x"], d["delta"], d["A"], d["B"], d["C"], D=d["D"], z=d["z"],
                                 delta_bias=d["delta_bias"], delta_softplus=softplus, h0=d["h0"],
                                 threads=ORACLE_THREADS)


def err(g, o):
    """max_i |g_i - o_i| / max(|o_i|, rms(o)): relative error with an rms floor
    (outputs where C.h + D.x cancels to ~0 carry only absolute rounding)."""
    g = np.asarray(g, np.float64)
    o = np.asarray(o, np.float64)
    if o.size == 0:
        return 0.0
    assert np.all(np.isfinite(g)), "non-finite GPU output"
    rms = float(np.sqrt(np.mean(o * o)))
    den = np.maximum(np.abs(o), rms if rms > 0 else 1e-300)
    return float(np.max(np.abs(g - o) / den))


def fp32_sequential(x, delta, A, B, C, D=None, z=None, delta_bias=None, softplus=True, h0=None):
    """The scan's definition evaluated step by step in fp32 (numpy float32,
    one rounding per operation; the decay applied as h + expm1(Delta A) h).
    Not a reference for parity -- the oracle is -- but the yardstick for what
    fp32 arithmetic itself loses on a given input: fp32 tests beyond the named
    workloads bound the kernel by this evaluation's own error (fp32_tolerance)."""
    f = np.float32
    x, delta = np.asarray(x, f), np.asarray(delta, f)
    Bt, T, Dd = x.shape
    A = np.asarray(A, f)
    N = A.shape[1]
    B, C = np.asarray(B, f), np.asarray(C, f)
    bias = np.zeros(Dd, f) if delta_bias is None else np.asarray(delta_bias, f)
    h = np.zeros((Bt, Dd, N), f) if h0 is None else np.array(h0, f)
    y = np.empty((Bt, T, Dd), np.float64)
    for t in range(T):
        v = (delta[:, t, :] + bias).astype(f)
        dt = (np.maximum(v, f(0)) + np.log1p(np.exp(-np.abs(v)))).astype(f) if softplus else v
        em = np.expm1((dt[:, :, None] * A[None]).astype(f)).astype(f)
        u = ((dt * x[:, t, :]).astype(f)[:, :, None] * B[:, t, None, :]).astype(f)
        h = ((em * h).astype(f) + h).astype(f)
        h = (h + u).astype(f)
        acc = np.zeros((Bt, Dd), f)
        for n in range(N):
            acc = (acc + (C[:, t, None, n] * h[:, :, n]).astype(f)).astype(f)
        if D is not None:
            acc = (acc + (np.asarray(D, f) * x[:, t, :]).astype(f)).astype(f)
        if z is not None:
            zz = np.asarray(z, f)[:, t, :]
            acc = (acc * (zz / (f(1) + np.exp(-zz)).astype(f)).astype(f)).astype(f)
        y[:, t, :] = acc
    return y, h.astype(np.float64)


def fp32_tolerance(o_y, o_last, **inputs):
    """1e-5, or 1.25 x the error a plain fp32 evaluation of the same inputs
    makes against the oracle when that is larger (long sequences over many
    channels: the max over millions of outputs of fp32's own rounding walk)."""
    y32, l32 = fp32_sequential(**inputs)
    e = max(err(y32, o_y), err(l32, o_last))
    return max(TOL[gen.F32], 1.25 * e), e