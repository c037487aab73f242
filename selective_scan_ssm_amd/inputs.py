"""Seeded synthetic inputs for the selective scan, shared by the tests, the
oracle checks and the benchmark.

This module holds no arithmetic of the scan itself: it only draws random
tensors with the shapes and distributions of the five workloads below and
stores them in the io dtype (fp32, or bf16 kept as raw uint16 bit patterns
because numpy has no bfloat16 type).

Distributions (same for every workload unless stated):
  x, z, delta      ~ N(0, 1) per (b, t, d)
  B, C             ~ N(0, 1) per (b, t, n), shared by every channel d
  delta_bias[d]    = log(expm1(dt_d)), dt_d log-uniform in [1e-3, 1e-1]
                     (the S4-style dt initialisation; softplus(bias) = dt)
  A[d, n]          = -(n + 1)          (the log(1..N) initialisation of A_log)
                     SM1 workload: A[d] = -exp(U(-4, 1))
  D[d]             ~ N(0, 1)
  h0               zero / N(0, 1) / absent, per workload
Each tensor comes from its own PCG64 stream, SeedSequence([seed, tensor_id]).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

F32 = "f32"
BF16 = "bf16"

# tensor ids inside one seed
_TID = {"x": 1, "delta": 2, "z": 3, "B": 4, "C": 5, "bias": 6, "A": 7, "D": 8, "h0": 9, "x_dbl": 10, "W_dt": 11,
        "conv_w": 12, "conv_b": 13, "conv_state": 14}


def bf16_from_f32(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 with round-to-nearest-even; returns uint16 bits.

    Finite inputs only (the generators never produce inf/nan)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    bits = a.view(np.uint32)
    lsb = (bits >> np.uint32(16)) & np.uint32(1)
    rounded = bits + np.uint32(0x7FFF) + lsb
    return (rounded >> np.uint32(16)).astype(np.uint16)


def f32_from_bf16(u: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to fp32."""
    u = np.ascontiguousarray(u, dtype=np.uint16)
    return (u.astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_f64(a: np.ndarray, io: str) -> np.ndarray:
    """Decode an io-dtype array (fp32, or bf16 bits) to fp64 exactly."""
    if io == BF16:
        return f32_from_bf16(a).astype(np.float64)
    return np.asarray(a, dtype=np.float32).astype(np.float64)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    seqlen: int
    d_inner: int
    d_state: int
    io: str
    a_kind: str          # "hippo" -> -(n+1); "sm1" -> -exp(U(-4,1)) per d
    h0_kind: str         # "zero", "normal", "none"
    kind: str = "scan"   # "scan", "sm1", "decode"
    layers: int = 1      # decode: independent layer states


WORKLOADS = {
    0: Workload("tiny-fp32", 1, 64, 16, 4, F32, "hippo", "zero"),
    1: Workload("sm1-fp32", 8, 4096, 1536, 1, F32, "sm1", "normal", kind="sm1"),
    2: Workload("mamba130m-layer-bf16", 8, 2048, 1536, 16, BF16, "hippo", "none"),
    3: Workload("mamba2.8b-layer-bf16", 4, 8192, 5120, 16, BF16, "hippo", "none"),
    4: Workload("decode-mamba2.8b-bf16", 256, 1, 5120, 16, BF16, "hippo", "normal",
                kind="decode", layers=64),
}


def _rng(seed: int, tensor: str, layer: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, _TID[tensor], layer])))


def _normal(seed, tensor, shape, layer=0) -> np.ndarray:
    return _rng(seed, tensor, layer).standard_normal(size=shape, dtype=np.float32)


def _store(a32: np.ndarray, io: str) -> np.ndarray:
    return bf16_from_f32(a32) if io == BF16 else np.ascontiguousarray(a32, dtype=np.float32)


def make_inputs(batch: int, seqlen: int, d_inner: int, d_state: int, io: str = F32,
                a_kind: str = "hippo", h0_kind: str = "zero", seed: int = 0,
                with_z: bool = True, with_D: bool = True, with_bias: bool = True,
                layer: int = 0) -> dict:
    """Draw one set of scan inputs.

    Returns a dict of numpy arrays: x, delta, z (B,T,D) and B, C (B,T,N) in the
    io dtype; A (D,N), D (D), delta_bias (D), h0 (B,D,N) in fp32.  Optional
    tensors are None when disabled.  For the SM1 layout (N = 1) the same
    arrays are used with the trailing N axis of size 1.
    """
    Bb, T, Dd, N = batch, seqlen, d_inner, d_state
    out = {"io": io, "batch": Bb, "seqlen": T, "d_inner": Dd, "d_state": N}
    out["x"] = _store(_normal(seed, "x", (Bb, T, Dd), layer), io)
    out["delta"] = _store(_normal(seed, "delta", (Bb, T, Dd), layer), io)
    out["z"] = _store(_normal(seed, "z", (Bb, T, Dd), layer), io) if with_z else None
    out["B"] = _store(_normal(seed, "B", (Bb, T, N), layer), io)
    out["C"] = _store(_normal(seed, "C", (Bb, T, N), layer), io)
    if with_bias:
        r = _rng(seed, "bias")
        dt = np.exp(r.uniform(np.log(1e-3), np.log(1e-1), size=Dd))
        out["delta_bias"] = np.log(np.expm1(dt)).astype(np.float32)
    else:
        out["delta_bias"] = None
    if a_kind == "hippo":
        out["A"] = np.ascontiguousarray(
            np.broadcast_to(-(np.arange(N, dtype=np.float32) + 1.0), (Dd, N)), dtype=np.float32)
    elif a_kind == "sm1":
        r = _rng(seed, "A")
        out["A"] = (-np.exp(r.uniform(-4.0, 1.0, size=(Dd, N)))).astype(np.float32)
    else:
        raise ValueError(a_kind)
    out["D"] = _normal(seed, "D", (Dd,)) if with_D else None
    if h0_kind == "zero":
        out["h0"] = np.zeros((Bb, Dd, N), dtype=np.float32)
    elif h0_kind == "normal":
        out["h0"] = _normal(seed, "h0", (Bb, Dd, N), layer)
    elif h0_kind == "none":
        out["h0"] = None
    else:
        raise ValueError(h0_kind)
    return out


def workload_inputs(cfg: int, seed: Optional[int] = None, layer: int = 0, **over) -> dict:
    """Inputs of one of the five named workloads (seed defaults to the workload id)."""
    w = WORKLOADS[cfg]
    kw = dict(batch=w.batch, seqlen=w.seqlen, d_inner=w.d_inner, d_state=w.d_state, io=w.io,
              a_kind=w.a_kind, h0_kind=w.h0_kind, seed=cfg if seed is None else seed, layer=layer)
    kw.update(over)
    return make_inputs(**kw)


# ------------------------------------------------------- the block's conv1d
# The causal depthwise conv1d in front of the scan (the guide's MambaBlock:
# nn.Conv1d(d_inner, d_inner, kernel_size=d_conv, groups=d_inner,
# padding=d_conv - 1)), with PyTorch's default initialisation of such a layer:
# weight and bias ~ U(-1/sqrt(K), 1/sqrt(K)) (fan-in K per channel).  The
# window before the sequence (for continuation) ~ N(0, 1) in the io dtype.
def make_conv_params(batch: int, d_inner: int, width: int, io: str = F32, seed: int = 0,
                     with_bias: bool = True, with_state: bool = False) -> dict:
    bound = 1.0 / np.sqrt(width)
    w = _rng(seed, "conv_w").uniform(-bound, bound, size=(d_inner, width)).astype(np.float32)
    b = _rng(seed, "conv_b").uniform(-bound, bound, size=d_inner).astype(np.float32) if with_bias else None
    st = _store(_normal(seed, "conv_state", (batch, d_inner, width - 1)), io) if with_state else None
    return {"conv_w": w, "conv_b": b, "conv_state": st}


# ------------------------------------------------------------- Mamba-2 (SSD)
# The multi-head scan of the youngju.dev guide's Mamba 2 section: the block is
# Mamba2Block(d_model, d_state=64, n_heads=8, chunk_size=64) with head size
# d_model / n_heads, one A_log per head drawn from N(0, 1), and an input
# projection that yields x and z (d_model each), B and C (d_state each, shared
# by the heads) and dt (one per head).
#   x, z, dt, B, C ~ N(0, 1)
#   A[h]          = -exp(A_log[h]), A_log[h] ~ N(0, 1)
#   dt_bias[h]    = log(expm1(dt_h)), dt_h log-uniform in [1e-3, 1e-1]
#   D[h]          ~ N(0, 1)
#   h0            zero / N(0, 1) / absent

@dataclasses.dataclass(frozen=True)
class SsdWorkload:
    name: str
    batch: int
    seqlen: int
    d_model: int
    n_heads: int
    d_state: int
    io: str
    h0_kind: str = "none"

    @property
    def headdim(self) -> int:
        return self.d_model // self.n_heads


SSD_WORKLOADS = {
    "mamba2-2.7b-ssd-layer-bf16": SsdWorkload("mamba2-2.7b-ssd-layer-bf16", 4, 8192, 2560, 8, 64, BF16),
    "mamba2-130m-ssd-layer-bf16": SsdWorkload("mamba2-130m-ssd-layer-bf16", 8, 2048, 768, 8, 64, BF16),
}


def make_ssd_inputs(batch: int, seqlen: int, nheads: int, headdim: int, d_state: int,
                    io: str = F32, h0_kind: str = "zero", seed: int = 0, with_z: bool = True,
                    with_D: bool = True, with_bias: bool = True) -> dict:
    """Draw one set of Mamba-2 scan inputs: x, z (B,T,H,P), dt (B,T,H), B, C
    (B,T,N) in the io dtype; A, D, dt_bias (H) and h0 (B,H,P,N) in fp32."""
    Bb, T, H, P, N = batch, seqlen, nheads, headdim, d_state
    out = {"io": io, "batch": Bb, "seqlen": T, "nheads": H, "headdim": P, "d_state": N}
    out["x"] = _store(_normal(seed, "x", (Bb, T, H, P)), io)
    out["dt"] = _store(_normal(seed, "delta", (Bb, T, H)), io)
    out["z"] = _store(_normal(seed, "z", (Bb, T, H, P)), io) if with_z else None
    out["B"] = _store(_normal(seed, "B", (Bb, T, N)), io)
    out["C"] = _store(_normal(seed, "C", (Bb, T, N)), io)
    if with_bias:
        r = _rng(seed, "bias")
        dtv = np.exp(r.uniform(np.log(1e-3), np.log(1e-1), size=H))
        out["dt_bias"] = np.log(np.expm1(dtv)).astype(np.float32)
    else:
        out["dt_bias"] = None
    out["A"] = (-np.exp(_normal(seed, "A", (H,)))).astype(np.float32)
    out["D"] = _normal(seed, "D", (H,)) if with_D else None
    if h0_kind == "zero":
        out["h0"] = np.zeros((Bb, H, P, N), dtype=np.float32)
    elif h0_kind == "normal":
        out["h0"] = _normal(seed, "h0", (Bb, H, P, N))
    elif h0_kind == "none":
        out["h0"] = None
    else:
        raise ValueError(h0_kind)
    return out


def ssd_workload_inputs(name: str, seed: int = 0, **over) -> dict:
    w = SSD_WORKLOADS[name]
    kw = dict(batch=w.batch, seqlen=w.seqlen, nheads=w.n_heads, headdim=w.headdim, d_state=w.d_state,
              io=w.io, h0_kind=w.h0_kind, seed=seed)
    kw.update(over)
    return make_ssd_inputs(**kw)


def make_dtproj_inputs(rows: int, rank: int, dim: int, ldx: int, io: str = BF16, seed: int = 0) -> dict:
    """Inputs of dt_proj (youngju.dev guide, section 5 MambaBlock: a linear
    layer dt_rank -> d_inner, dt_init "random" with dt_scale 1): x_dbl
    (rows, ldx), the x_proj output whose first `rank` columns are the dt input
    and the rest (B, C) are not read, ~ N(0, 1); W (dim, rank) ~ U(-s, s) with
    s = rank^-1/2, the layer's random init.  Both stored in the io dtype."""
    out = {"io": io, "rows": rows, "rank": rank, "dim": dim, "ldx": ldx}
    out["x_dbl"] = _store(_normal(seed, "x_dbl", (rows, ldx)), io)
    s = rank ** -0.5
    out["W"] = _store(_rng(seed, "W_dt").uniform(-s, s, size=(dim, rank)).astype(np.float32), io)
    return out
