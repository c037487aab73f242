"""Thin torch-facing wrappers of the C ABI (include/ssm_scan.h).

They only marshal arguments: check devices, dtypes, shapes and contiguity,
allocate outputs (and the workspace) with torch, pass raw device pointers and
torch's current HIP stream to libssmscan.so, and turn a nonzero status into
RuntimeError.  Every step of the computation runs in the library's kernels.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import _lib

_IO = {torch.float32: _lib.SSM_F32, torch.bfloat16: _lib.SSM_BF16}


def _check(rc: int, what: str):
    if rc != 0:
        raise RuntimeError(f"{what}: {_lib.status_string(rc)}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _dev(t: torch.Tensor, name: str, dtype=None, shape=None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def scan_fwd(x, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=True, h0=None,
             return_last_state=False, out=None, last_state_out=None, workspace=None, ckpt_out=None):
    """Selective scan.  x, delta, z: (batch, seqlen, d_inner) fp32 or bf16;
    B, C: (batch, seqlen, d_state) same dtype; A: (d_inner, d_state) fp32;
    D, delta_bias: (d_inner,) fp32; h0: (batch, d_inner, d_state) fp32.
    Returns y (same dtype as x) or (y, last_state fp32).  ckpt_out: an fp32
    tensor of ckpt_shape(...) that also receives the state entering every
    16-step block (ssm_scan_fwd_ckpt), for scan_bwd(..., ckpt=ckpt_out)."""
    lib = _lib.load()
    if x.dtype not in _IO:
        raise ValueError("x must be float32 or bfloat16")
    io = x.dtype
    Bt, T, Dd = x.shape
    N = A.shape[-1]
    _dev(x, "x", io)
    _dev(delta, "delta", io, x.shape)
    _dev(z, "z", io, x.shape)
    _dev(B, "B", io, (Bt, T, N))
    _dev(C, "C", io, (Bt, T, N))
    _dev(A, "A", torch.float32, (Dd, N))
    _dev(D, "D", torch.float32, (Dd,))
    _dev(delta_bias, "delta_bias", torch.float32, (Dd,))
    _dev(h0, "h0", torch.float32, (Bt, Dd, N))
    y = out if out is not None else torch.empty_like(x)
    _dev(y, "out", io, x.shape)
    last = None
    if return_last_state:
        last = last_state_out if last_state_out is not None else torch.empty(
            (Bt, Dd, N), dtype=torch.float32, device=x.device)
        _dev(last, "last_state_out", torch.float32, (Bt, Dd, N))
    need = lib.ssm_scan_workspace_bytes(Bt, T, Dd, N, _IO[io])
    if need == (1 << 64) - 1:
        raise RuntimeError("ssm_scan_workspace_bytes: invalid arguments")
    ws = None
    if need:
        ws = workspace if workspace is not None and workspace.numel() >= need else torch.empty(
            need, dtype=torch.uint8, device=x.device)
    if ckpt_out is not None:
        _dev(ckpt_out, "ckpt_out", torch.float32, ckpt_shape(Bt, T, Dd, N))
        rc = lib.ssm_scan_fwd_ckpt(_ptr(x), _ptr(delta), _ptr(delta_bias), int(bool(delta_softplus)),
                                   _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(h0), _ptr(y), _ptr(last),
                                   _ptr(ckpt_out), Bt, T, Dd, N, _IO[io], _ptr(ws), need, _stream(x.device))
        _check(rc, "ssm_scan_fwd_ckpt")
    else:
        rc = lib.ssm_scan_fwd(_ptr(x), _ptr(delta), _ptr(delta_bias), int(bool(delta_softplus)),
                              _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(h0), _ptr(y), _ptr(last),
                              Bt, T, Dd, N, _IO[io], _ptr(ws), need, _stream(x.device))
        _check(rc, "ssm_scan_fwd")
    return (y, last) if return_last_state else y


def ckpt_shape(batch, seqlen, d_inner, d_state):
    """Shape of the saved checkpoints: (batch, ceil(seqlen / 16), d_inner, d_state)."""
    return (batch, (seqlen + 15) // 16, d_inner, d_state)


def sm1_scan_fwd(x, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=True, h0=None,
                 return_last_state=False, out=None, last_state_out=None, workspace=None):
    """d_state = 1 scan.  x, delta, z: (batch, seqlen, d_inner); B, C: (batch, seqlen);
    A, D, delta_bias: (d_inner,); h0, last_state: (batch, d_inner)."""
    lib = _lib.load()
    if x.dtype not in _IO:
        raise ValueError("x must be float32 or bfloat16")
    io = x.dtype
    Bt, T, Dd = x.shape
    _dev(x, "x", io)
    _dev(delta, "delta", io, x.shape)
    _dev(z, "z", io, x.shape)
    _dev(B, "B", io, (Bt, T))
    _dev(C, "C", io, (Bt, T))
    _dev(A, "A", torch.float32, (Dd,))
    _dev(D, "D", torch.float32, (Dd,))
    _dev(delta_bias, "delta_bias", torch.float32, (Dd,))
    _dev(h0, "h0", torch.float32, (Bt, Dd))
    y = out if out is not None else torch.empty_like(x)
    _dev(y, "out", io, x.shape)
    last = None
    if return_last_state:
        last = last_state_out if last_state_out is not None else torch.empty(
            (Bt, Dd), dtype=torch.float32, device=x.device)
        _dev(last, "last_state_out", torch.float32, (Bt, Dd))
    need = lib.sm1_scan_workspace_bytes(Bt, T, Dd, _IO[io])
    if need == (1 << 64) - 1:
        raise RuntimeError("sm1_scan_workspace_bytes: invalid arguments")
    ws = None
    if need:
        ws = workspace if workspace is not None and workspace.numel() >= need else torch.empty(
            need, dtype=torch.uint8, device=x.device)
    rc = lib.sm1_scan_fwd(_ptr(x), _ptr(delta), _ptr(delta_bias), int(bool(delta_softplus)),
                          _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(h0), _ptr(y), _ptr(last),
                          Bt, T, Dd, _IO[io], _ptr(ws), need, _stream(x.device))
    _check(rc, "sm1_scan_fwd")
    return (y, last) if return_last_state else y


def state_update(state, x, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=True,
                 out=None):
    """One decode step; `state` (batch, d_inner, d_state) fp32 is updated in place.
    x, delta, z: (batch, d_inner); B, C: (batch, d_state).  Returns y."""
    lib = _lib.load()
    if x.dtype not in _IO:
        raise ValueError("x must be float32 or bfloat16")
    io = x.dtype
    Bt, Dd = x.shape
    N = A.shape[-1]
    _dev(state, "state", torch.float32, (Bt, Dd, N))
    _dev(x, "x", io)
    _dev(delta, "delta", io, x.shape)
    _dev(z, "z", io, x.shape)
    _dev(B, "B", io, (Bt, N))
    _dev(C, "C", io, (Bt, N))
    _dev(A, "A", torch.float32, (Dd, N))
    _dev(D, "D", torch.float32, (Dd,))
    _dev(delta_bias, "delta_bias", torch.float32, (Dd,))
    y = out if out is not None else torch.empty_like(x)
    _dev(y, "out", io, x.shape)
    rc = lib.ssm_state_update(_ptr(state), _ptr(x), _ptr(delta), _ptr(delta_bias),
                              int(bool(delta_softplus)), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                              _ptr(y), Bt, Dd, N, _IO[io], _stream(x.device))
    _check(rc, "ssm_state_update")
    return y


def scan_bwd(x, delta, A, B, C, dout, D=None, z=None, delta_bias=None, delta_softplus=True,
             h0=None, dlast=None, workspace=None, ckpt=None):
    """Gradient of `scan_fwd`.  Same inputs, plus dout = dL/dy (like x) and
    dlast = dL/dlast_state ((batch, d_inner, d_state) fp32, optional).  Returns
    a dict: dx, ddelta, dB, dC (dtype of x), dA, dh0 (fp32), and dz, dD,
    ddelta_bias (fp32 for dD / ddelta_bias) when z, D, delta_bias are given.
    ckpt: the checkpoints scan_fwd(..., ckpt_out=) recorded on the same inputs
    (ssm_scan_bwd_ckpt); the backward then skips its own checkpoint pass."""
    lib = _lib.load()
    if x.dtype not in _IO:
        raise ValueError("x must be float32 or bfloat16")
    io = x.dtype
    Bt, T, Dd = x.shape
    N = A.shape[-1]
    _dev(x, "x", io)
    _dev(delta, "delta", io, x.shape)
    _dev(z, "z", io, x.shape)
    _dev(dout, "dout", io, x.shape)
    _dev(B, "B", io, (Bt, T, N))
    _dev(C, "C", io, (Bt, T, N))
    _dev(A, "A", torch.float32, (Dd, N))
    _dev(D, "D", torch.float32, (Dd,))
    _dev(delta_bias, "delta_bias", torch.float32, (Dd,))
    _dev(h0, "h0", torch.float32, (Bt, Dd, N))
    _dev(dlast, "dlast", torch.float32, (Bt, Dd, N))
    dev = x.device
    g = dict(dx=torch.empty_like(x), ddelta=torch.empty_like(x), dB=torch.empty_like(B),
             dC=torch.empty_like(C), dA=torch.empty((Dd, N), dtype=torch.float32, device=dev),
             dh0=torch.empty((Bt, Dd, N), dtype=torch.float32, device=dev),
             dz=torch.empty_like(x) if z is not None else None,
             dD=torch.empty((Dd,), dtype=torch.float32, device=dev) if D is not None else None,
             ddelta_bias=torch.empty((Dd,), dtype=torch.float32, device=dev) if delta_bias is not None else None)
    need = lib.ssm_scan_bwd_workspace_bytes(Bt, T, Dd, N, _IO[io])
    if need == (1 << 64) - 1:
        raise RuntimeError("ssm_scan_bwd_workspace_bytes: invalid arguments")
    ws = None
    if need:
        ws = workspace if workspace is not None and workspace.numel() >= need else torch.empty(
            need, dtype=torch.uint8, device=dev)
    outs = (_ptr(g["dx"]), _ptr(g["ddelta"]), _ptr(g["ddelta_bias"]), _ptr(g["dA"]), _ptr(g["dB"]),
            _ptr(g["dC"]), _ptr(g["dD"]), _ptr(g["dz"]), _ptr(g["dh0"]))
    if ckpt is not None:
        _dev(ckpt, "ckpt", torch.float32, ckpt_shape(Bt, T, Dd, N))
        rc = lib.ssm_scan_bwd_ckpt(_ptr(x), _ptr(delta), _ptr(delta_bias), int(bool(delta_softplus)),
                                   _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(h0), _ptr(dout),
                                   _ptr(dlast), _ptr(ckpt), *outs, Bt, T, Dd, N, _IO[io], _ptr(ws), need,
                                   _stream(dev))
        _check(rc, "ssm_scan_bwd_ckpt")
    else:
        rc = lib.ssm_scan_bwd(_ptr(x), _ptr(delta), _ptr(delta_bias), int(bool(delta_softplus)),
                              _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(h0), _ptr(dout),
                              _ptr(dlast), *outs, Bt, T, Dd, N, _IO[io], _ptr(ws), need, _stream(dev))
        _check(rc, "ssm_scan_bwd")
    return g


def dt_proj(xdt, W, out=None):
    """delta = xdt @ W.T, the Mamba block's dt_proj without its bias (the bias
    is the scan's delta_bias).  xdt: (rows, rank) or (batch, seqlen, rank),
    fp32 or bf16, whose last axis is contiguous and whose rows are evenly
    strided: typically the first rank columns of the x_proj output, a view.
    W: (d_inner, rank) in the same dtype.  Returns delta (..., d_inner)."""
    lib = _lib.load()
    if xdt.dtype not in _IO:
        raise ValueError("xdt must be float32 or bfloat16")
    io = xdt.dtype
    if xdt.dim() not in (2, 3) or (xdt.shape[-1] > 1 and xdt.stride(-1) != 1):
        raise ValueError("xdt must be 2-D or 3-D with a contiguous last axis")
    rank = xdt.shape[-1]
    rows = xdt.numel() // rank if rank else 0
    # the stride between consecutive rows, from the leading axes of size > 1
    # (torch may report any stride for an axis of size 1)
    lead = [(n, st) for n, st in zip(xdt.shape[:-1], xdt.stride()[:-1]) if n > 1]
    if len(lead) == 2 and lead[0][1] != lead[1][0] * lead[1][1]:
        raise ValueError("the rows of xdt must be evenly strided")
    ldx = lead[-1][1] if lead else rank
    Dd = W.shape[0]
    if not xdt.is_cuda:
        raise ValueError("xdt must be a GPU tensor")
    _dev(W, "W", io, (Dd, rank))
    y = out if out is not None else torch.empty(tuple(xdt.shape[:-1]) + (Dd,), dtype=io, device=xdt.device)
    _dev(y, "out", io, tuple(xdt.shape[:-1]) + (Dd,))
    rc = lib.ssm_dt_proj(_ptr(xdt), ldx, _ptr(W), _ptr(y), rows, rank, Dd, _IO[io], _stream(xdt.device))
    _check(rc, "ssm_dt_proj")
    return y


def causal_conv1d(x, weight, bias=None, conv_state=None, silu=True, return_state=False, out=None):
    """Causal depthwise conv1d (+ SiLU) of the Mamba block's x branch.
    x: (batch, seqlen, d_inner) fp32 or bf16; weight: (d_inner, width) fp32;
    bias: (d_inner,) fp32; conv_state: (batch, d_inner, width - 1) like x, the
    inputs before the sequence.  Returns out, or (out, new conv_state)."""
    lib = _lib.load()
    if x.dtype not in _IO:
        raise ValueError("x must be float32 or bfloat16")
    io = x.dtype
    Bt, T, Dd = x.shape
    K = weight.shape[-1]
    _dev(x, "x", io)
    _dev(weight, "weight", torch.float32, (Dd, K))
    _dev(bias, "bias", torch.float32, (Dd,))
    _dev(conv_state, "conv_state", io, (Bt, Dd, K - 1))
    y = out if out is not None else torch.empty_like(x)
    _dev(y, "out", io, x.shape)
    st = torch.empty((Bt, Dd, K - 1), dtype=io, device=x.device) if return_state else None
    rc = lib.ssm_causal_conv1d_fwd(_ptr(x), _ptr(weight), _ptr(bias), _ptr(conv_state), _ptr(y),
                                   _ptr(st), int(bool(silu)), Bt, T, Dd, K, _IO[io], _stream(x.device))
    _check(rc, "ssm_causal_conv1d_fwd")
    return (y, st) if return_state else y


def causal_conv1d_update(conv_state, x, weight, bias=None, silu=True, out=None):
    """One decode token: conv_state (batch, d_inner, width - 1) is updated in
    place; x: (batch, d_inner).  Returns out (batch, d_inner)."""
    lib = _lib.load()
    if x.dtype not in _IO:
        raise ValueError("x must be float32 or bfloat16")
    io = x.dtype
    Bt, Dd = x.shape
    K = weight.shape[-1]
    _dev(conv_state, "conv_state", io, (Bt, Dd, K - 1))
    _dev(x, "x", io)
    _dev(weight, "weight", torch.float32, (Dd, K))
    _dev(bias, "bias", torch.float32, (Dd,))
    y = out if out is not None else torch.empty_like(x)
    _dev(y, "out", io, x.shape)
    rc = lib.ssm_causal_conv1d_update(_ptr(conv_state), _ptr(x), _ptr(weight), _ptr(bias), _ptr(y),
                                      int(bool(silu)), Bt, Dd, K, _IO[io], _stream(x.device))
    _check(rc, "ssm_causal_conv1d_update")
    return y


def scan_fwd_2d(x, delta, A, B, C, height, width, direction, D=None, z=None, delta_bias=None,
                delta_softplus=True, h0=None, return_last_state=False, out=None, workspace=None):
    """One direction (0 row-major, 1 reverse, 2 column-major, 3 reverse
    column-major) of the 2-D scan over height x width patches held row-major
    on the sequence axis; y comes back at each patch's position."""
    lib = _lib.load()
    if x.dtype not in _IO:
        raise ValueError("x must be float32 or bfloat16")
    io = x.dtype
    Bt, T, Dd = x.shape
    N = A.shape[-1]
    if T != height * width:
        raise ValueError("seqlen must be height * width")
    _dev(x, "x", io)
    _dev(delta, "delta", io, x.shape)
    _dev(z, "z", io, x.shape)
    _dev(B, "B", io, (Bt, T, N))
    _dev(C, "C", io, (Bt, T, N))
    _dev(A, "A", torch.float32, (Dd, N))
    _dev(D, "D", torch.float32, (Dd,))
    _dev(delta_bias, "delta_bias", torch.float32, (Dd,))
    _dev(h0, "h0", torch.float32, (Bt, Dd, N))
    y = out if out is not None else torch.empty_like(x)
    _dev(y, "out", io, x.shape)
    last = torch.empty((Bt, Dd, N), dtype=torch.float32, device=x.device) if return_last_state else None
    need = lib.ssm_scan_2d_workspace_bytes(Bt, height, width, Dd, N, int(direction), int(z is not None), _IO[io])
    if need == (1 << 64) - 1:
        raise RuntimeError("ssm_scan_2d_workspace_bytes: invalid arguments")
    ws = None
    if need:
        ws = workspace if workspace is not None and workspace.numel() >= need else torch.empty(
            need, dtype=torch.uint8, device=x.device)
    rc = lib.ssm_scan_fwd_2d(_ptr(x), _ptr(delta), _ptr(delta_bias), int(bool(delta_softplus)),
                             _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(h0), _ptr(y), _ptr(last),
                             Bt, height, width, Dd, N, int(direction), _IO[io], _ptr(ws), need,
                             _stream(x.device))
    _check(rc, "ssm_scan_fwd_2d")
    return (y, last) if return_last_state else y


def ssd_scan_fwd(x, dt, A, B, C, D=None, z=None, dt_bias=None, dt_softplus=True, h0=None,
                 return_last_state=False, out=None, last_state_out=None, workspace=None):
    """Mamba-2 multi-head scan.  x, z: (batch, seqlen, nheads, headdim) fp32 or
    bf16; dt: (batch, seqlen, nheads); B, C: (batch, seqlen, dstate) same dtype;
    A, D, dt_bias: (nheads,) fp32; h0: (batch, nheads, headdim, dstate) fp32.
    Returns y (same dtype as x) or (y, last_state fp32)."""
    lib = _lib.load()
    if x.dtype not in _IO:
        raise ValueError("x must be float32 or bfloat16")
    io = x.dtype
    Bt, T, H, P = x.shape
    N = B.shape[-1]
    _dev(x, "x", io)
    _dev(dt, "dt", io, (Bt, T, H))
    _dev(z, "z", io, x.shape)
    _dev(B, "B", io, (Bt, T, N))
    _dev(C, "C", io, (Bt, T, N))
    _dev(A, "A", torch.float32, (H,))
    _dev(D, "D", torch.float32, (H,))
    _dev(dt_bias, "dt_bias", torch.float32, (H,))
    _dev(h0, "h0", torch.float32, (Bt, H, P, N))
    y = out if out is not None else torch.empty_like(x)
    _dev(y, "out", io, x.shape)
    last = None
    if return_last_state:
        last = last_state_out if last_state_out is not None else torch.empty(
            (Bt, H, P, N), dtype=torch.float32, device=x.device)
        _dev(last, "last_state_out", torch.float32, (Bt, H, P, N))
    need = lib.ssd_scan_workspace_bytes(Bt, T, H, P, N, _IO[io])
    if need == (1 << 64) - 1:
        raise RuntimeError("ssd_scan_workspace_bytes: invalid arguments")
    ws = None
    if need:
        ws = workspace if workspace is not None and workspace.numel() >= need else torch.empty(
            need, dtype=torch.uint8, device=x.device)
    rc = lib.ssd_scan_fwd(_ptr(x), _ptr(dt), _ptr(dt_bias), int(bool(dt_softplus)), _ptr(A), _ptr(B),
                          _ptr(C), _ptr(D), _ptr(z), _ptr(h0), _ptr(y), _ptr(last), Bt, T, H, P, N,
                          _IO[io], _ptr(ws), need, _stream(x.device))
    _check(rc, "ssd_scan_fwd")
    return (y, last) if return_last_state else y


def scan_status(workspace, stream_device=None):
    """ssm_scan_status on a workspace tensor (uint8, device) of the last
    forward scan: 0 (SSM_OK) or SSM_ERR_WAIT when a segment's bounded wait
    gave up.  Synchronises torch's current stream of the workspace's device."""
    lib = _lib.load()
    dev = workspace.device if stream_device is None else stream_device
    return lib.ssm_scan_status(_ptr(workspace), workspace.numel(), _stream(dev))


def scan_workspace_bytes(batch, seqlen, d_inner, d_state, dtype):
    """ssm_scan_workspace_bytes for io dtype `dtype` (torch.float32 / torch.bfloat16)."""
    need = _lib.load().ssm_scan_workspace_bytes(batch, seqlen, d_inner, d_state, _IO[dtype])
    if need == (1 << 64) - 1:
        raise RuntimeError("ssm_scan_workspace_bytes: invalid arguments")
    return need


def conv_scan_fwd(x, conv_weight, delta, A, B, C, conv_bias=None, conv_state=None, D=None, z=None,
                  delta_bias=None, delta_softplus=True, h0=None, return_last_state=False,
                  return_conv_state=False, out=None, workspace=None):
    """The block's prologue and the scan in one call (ssm_conv_scan_fwd): the
    scan of scan_fwd on SiLU(causal_conv1d(x)).  x: (batch, seqlen, d_inner)
    conv input; conv_weight: (d_inner, width) fp32; conv_bias: (d_inner,)
    fp32; conv_state: (batch, d_inner, width - 1) in x's dtype.  Returns y,
    plus last_state and/or the conv window after the sequence when asked."""
    lib = _lib.load()
    if x.dtype not in _IO:
        raise ValueError("x must be float32 or bfloat16")
    io = x.dtype
    Bt, T, Dd = x.shape
    N = A.shape[-1]
    K = conv_weight.shape[-1]
    _dev(x, "x", io)
    _dev(conv_weight, "conv_weight", torch.float32, (Dd, K))
    _dev(conv_bias, "conv_bias", torch.float32, (Dd,))
    _dev(conv_state, "conv_state", io, (Bt, Dd, K - 1))
    _dev(delta, "delta", io, x.shape)
    _dev(z, "z", io, x.shape)
    _dev(B, "B", io, (Bt, T, N))
    _dev(C, "C", io, (Bt, T, N))
    _dev(A, "A", torch.float32, (Dd, N))
    _dev(D, "D", torch.float32, (Dd,))
    _dev(delta_bias, "delta_bias", torch.float32, (Dd,))
    _dev(h0, "h0", torch.float32, (Bt, Dd, N))
    y = out if out is not None else torch.empty_like(x)
    _dev(y, "out", io, x.shape)
    last = torch.empty((Bt, Dd, N), dtype=torch.float32, device=x.device) if return_last_state else None
    win = torch.empty((Bt, Dd, K - 1), dtype=io, device=x.device) if return_conv_state else None
    need = lib.ssm_conv_scan_workspace_bytes(Bt, T, Dd, N, _IO[io])
    if need == (1 << 64) - 1:
        raise RuntimeError("ssm_conv_scan_workspace_bytes: invalid arguments")
    ws = None
    if need:
        ws = workspace if workspace is not None and workspace.numel() >= need else torch.empty(
            need, dtype=torch.uint8, device=x.device)
    rc = lib.ssm_conv_scan_fwd(_ptr(x), _ptr(conv_weight), _ptr(conv_bias), _ptr(conv_state), _ptr(win), K,
                               _ptr(delta), _ptr(delta_bias), int(bool(delta_softplus)), _ptr(A), _ptr(B),
                               _ptr(C), _ptr(D), _ptr(z), _ptr(h0), _ptr(y), _ptr(last), Bt, T, Dd, N, _IO[io],
                               _ptr(ws), need, _stream(x.device))
    _check(rc, "ssm_conv_scan_fwd")
    res = (y,)
    if return_last_state:
        res += (last,)
    if return_conv_state:
        res += (win,)
    return res if len(res) > 1 else y
