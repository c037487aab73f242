"""Python front end of the fp64 CPU oracle (ssm_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the GPU library or its binding.

`build()` compiles ssm_oracle.c with gcc; the wrappers take numpy arrays of
any float dtype, widen them to fp64 (exact for fp32 and for bf16 already
decoded to fp32/fp64), and call the C code, optionally on several threads
over disjoint ranges of (b, d) chains.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssm_oracle.c")
_BUILD_DIR = os.path.join(_HERE, "_build")
_LIB_PATH = os.path.join(_BUILD_DIR, "libssm_oracle.so")
# a sanitized build (build_sanitized) is loaded instead when this names it
_LIB_OVERRIDE = os.environ.get("SSM_ORACLE_LIB")
_lib = None
_lock = threading.Lock()

# strict IEEE fp64: no fast-math, no contraction into fma
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math", "-ffp-contract=off"]


def build(src: str = _SRC, out: str = _LIB_PATH) -> str:
    """Compile the oracle C source into a shared library; returns its path."""
    os.makedirs(os.path.dirname(out), exist_ok=True)
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.run(["gcc", *CFLAGS, src, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, out)
    return out


def build_sanitized(out: str, cc: str = "clang") -> str:
    """The same source and fp flags under AddressSanitizer and
    UndefinedBehaviorSanitizer (any report aborts), for the CPU check that
    runs the oracle's pins against it."""
    os.makedirs(os.path.dirname(out), exist_ok=True)
    subprocess.run([cc, *CFLAGS, "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-shared-libasan", _SRC, "-o", out, "-lm"], check=True)
    return out


_dp = ctypes.POINTER(ctypes.c_double)
_L = ctypes.c_long


def _bind(lib):
    lib.oracle_selective_scan.argtypes = [_dp, _dp, _dp, ctypes.c_int, _dp, _dp, _dp, _dp, _dp,
                                          _dp, _dp, _dp, _L, _L, _L, _L, _L, _L]
    lib.oracle_selective_scan.restype = None
    lib.oracle_state_update.argtypes = [_dp, _dp, _dp, _dp, ctypes.c_int, _dp, _dp, _dp, _dp,
                                        _dp, _dp, _L, _L, _L, _L, _L]
    lib.oracle_state_update.restype = None
    lib.oracle_sm1_scan.argtypes = [_dp, _dp, _dp, ctypes.c_int, _dp, _dp, _dp, _dp, _dp, _dp,
                                    _dp, _dp, _L, _L, _L, _L, _L]
    lib.oracle_sm1_scan.restype = None
    lib.oracle_selective_scan_bwd.argtypes = [_dp, _dp, _dp, ctypes.c_int, _dp, _dp, _dp, _dp, _dp,
                                              _dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp,
                                              _dp, _dp, _L, _L, _L, _L, _L, _L]
    lib.oracle_selective_scan_bwd.restype = None
    lib.oracle_causal_conv1d.argtypes = [_dp, _dp, _dp, _dp, _dp, _dp, ctypes.c_int,
                                         _L, _L, _L, _L, _L, _L]
    lib.oracle_causal_conv1d.restype = None
    lib.oracle_conv1d_update.argtypes = [_dp, _dp, _dp, _dp, _dp, ctypes.c_int, _L, _L, _L, _L, _L]
    lib.oracle_conv1d_update.restype = None
    lib.oracle_dt_proj.argtypes = [_dp, _L, _dp, _dp, _L, _L, _L, _L, _L]
    lib.oracle_ssd_scan.argtypes = [_dp, _dp, _dp, ctypes.c_int, _dp, _dp, _dp, _dp, _dp, _dp,
                                    _dp, _dp, _L, _L, _L, _L, _L, _L, _L]
    lib.oracle_ssd_scan.restype = None
    return lib


def load(path: Optional[str] = None):
    """Load (building first if needed) the oracle library."""
    global _lib
    with _lock:
        if path is not None:
            return _bind(ctypes.CDLL(path))
        if _lib is None and _LIB_OVERRIDE:
            _lib = _bind(ctypes.CDLL(_LIB_OVERRIDE))
        if _lib is None:
            if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
                build()
            _lib = _bind(ctypes.CDLL(_LIB_PATH))
        return _lib


def _f64(a):
    if a is None:
        return None
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a):
    if a is None:
        return ctypes.cast(None, _dp)
    return a.ctypes.data_as(_dp)


def _run_chains(fn, n_chains: int, threads: int):
    threads = max(1, min(int(threads), n_chains if n_chains > 0 else 1))
    if threads == 1:
        fn(0, n_chains)
        return
    step = (n_chains + threads - 1) // threads
    ts = [threading.Thread(target=fn, args=(i, min(i + step, n_chains)))
          for i in range(0, n_chains, step)]
    for t in ts:
        t.start()
    for t in ts:
        t.join()


def selective_scan(x, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=True,
                   h0=None, threads: int = 1, lib=None):
    """Sequential fp64 scan.  x, delta, z: (Bt, T, Dd); B, C: (Bt, T, N); A: (Dd, N);
    D, delta_bias: (Dd,); h0: (Bt, Dd, N).  Returns (y, last_state) in fp64."""
    lib = lib or load()
    x, delta, A, B, C = _f64(x), _f64(delta), _f64(A), _f64(B), _f64(C)
    D, z, delta_bias, h0 = _f64(D), _f64(z), _f64(delta_bias), _f64(h0)
    Bt, T, Dd = x.shape
    N = A.shape[1]
    assert delta.shape == x.shape and A.shape == (Dd, N)
    assert B.shape == (Bt, T, N) and C.shape == (Bt, T, N)
    assert z is None or z.shape == x.shape
    assert h0 is None or h0.shape == (Bt, Dd, N)
    y = np.zeros((Bt, T, Dd), dtype=np.float64)
    last = np.zeros((Bt, Dd, N), dtype=np.float64)

    def go(c0, c1):
        lib.oracle_selective_scan(_ptr(x), _ptr(delta), _ptr(delta_bias), int(bool(delta_softplus)),
                                  _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(h0),
                                  _ptr(y), _ptr(last), Bt, T, Dd, N, c0, c1)

    _run_chains(go, Bt * Dd, threads)
    return y, last


def state_update(state, x, delta, A, B, C, D=None, z=None, delta_bias=None,
                 delta_softplus=True, threads: int = 1, lib=None):
    """One decode step.  state: (Bt, Dd, N) (not modified; the new state is
    returned); x, delta, z: (Bt, Dd); B, C: (Bt, N).  Returns (y, new_state)."""
    lib = lib or load()
    st = _f64(state).copy()
    x, delta, A, B, C = _f64(x), _f64(delta), _f64(A), _f64(B), _f64(C)
    D, z, delta_bias = _f64(D), _f64(z), _f64(delta_bias)
    Bt, Dd = x.shape
    N = A.shape[1]
    assert st.shape == (Bt, Dd, N) and B.shape == (Bt, N) and C.shape == (Bt, N)
    y = np.zeros((Bt, Dd), dtype=np.float64)

    def go(c0, c1):
        lib.oracle_state_update(_ptr(st), _ptr(x), _ptr(delta), _ptr(delta_bias),
                                int(bool(delta_softplus)), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                                _ptr(z), _ptr(y), Bt, Dd, N, c0, c1)

    _run_chains(go, Bt * Dd, threads)
    return y, st


def sm1_scan(x, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=True,
             h0=None, threads: int = 1, lib=None):
    """d_state = 1 scan.  A: (Dd,); B, C: (Bt, T); h0: (Bt, Dd).  Returns
    (y (Bt,T,Dd), last_state (Bt,Dd))."""
    lib = lib or load()
    x, delta, A, B, C = _f64(x), _f64(delta), _f64(A), _f64(B), _f64(C)
    D, z, delta_bias, h0 = _f64(D), _f64(z), _f64(delta_bias), _f64(h0)
    Bt, T, Dd = x.shape
    assert A.shape == (Dd,) and B.shape == (Bt, T) and C.shape == (Bt, T)
    assert h0 is None or h0.shape == (Bt, Dd)
    y = np.zeros((Bt, T, Dd), dtype=np.float64)
    last = np.zeros((Bt, Dd), dtype=np.float64)

    def go(c0, c1):
        lib.oracle_sm1_scan(_ptr(x), _ptr(delta), _ptr(delta_bias), int(bool(delta_softplus)),
                            _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(h0), _ptr(y),
                            _ptr(last), Bt, T, Dd, c0, c1)

    _run_chains(go, Bt * Dd, threads)
    return y, last


def selective_scan_bwd(x, delta, A, B, C, dout, D=None, z=None, delta_bias=None,
                       delta_softplus=True, h0=None, dlast=None, threads: int = 1, lib=None):
    """fp64 gradient of `selective_scan` (ssm_oracle.c, oracle_selective_scan_bwd).
    dout: (Bt, T, Dd) = dL/dy; dlast: (Bt, Dd, N) = dL/dlast_state or None.
    Returns a dict with dx, ddelta (Bt,T,Dd), dA (Dd,N), dB, dC (Bt,T,N),
    dh0 (Bt,Dd,N), and dD, ddelta_bias (Dd,), dz (Bt,T,Dd) when the forward
    had D, delta_bias, z (else None).  Threads accumulate the summed gradients
    into separate arrays, added in thread order."""
    lib = lib or load()
    x, delta, A, B, C, dout = _f64(x), _f64(delta), _f64(A), _f64(B), _f64(C), _f64(dout)
    D, z, delta_bias, h0, dlast = _f64(D), _f64(z), _f64(delta_bias), _f64(h0), _f64(dlast)
    Bt, T, Dd = x.shape
    N = A.shape[1]
    assert delta.shape == x.shape and dout.shape == x.shape and A.shape == (Dd, N)
    assert B.shape == (Bt, T, N) and C.shape == (Bt, T, N)
    assert z is None or z.shape == x.shape
    assert h0 is None or h0.shape == (Bt, Dd, N)
    assert dlast is None or dlast.shape == (Bt, Dd, N)
    dx = np.zeros_like(x)
    ddelta = np.zeros_like(x)
    dz = np.zeros_like(x) if z is not None else None
    dh0 = np.zeros((Bt, Dd, N))
    n_chains = Bt * Dd
    nthr = max(1, min(int(threads), n_chains if n_chains > 0 else 1))
    step = (n_chains + nthr - 1) // nthr if n_chains > 0 else 1
    ranges = [(c0, min(c0 + step, n_chains)) for c0 in range(0, max(n_chains, 1), step)]
    acc = [dict(dA=np.zeros((Dd, N)), dB=np.zeros((Bt, T, N)), dC=np.zeros((Bt, T, N)),
                dD=np.zeros(Dd), dbias=np.zeros(Dd)) for _ in ranges]

    def go(i):
        c0, c1 = ranges[i]
        a = acc[i]
        lib.oracle_selective_scan_bwd(_ptr(x), _ptr(delta), _ptr(delta_bias), int(bool(delta_softplus)),
                                      _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(h0),
                                      _ptr(dout), _ptr(dlast), _ptr(dx), _ptr(ddelta),
                                      _ptr(a["dbias"]), _ptr(a["dA"]), _ptr(a["dB"]), _ptr(a["dC"]),
                                      _ptr(a["dD"]), _ptr(dz), _ptr(dh0), Bt, T, Dd, N, c0, c1)

    if len(ranges) == 1:
        go(0)
    else:
        ts = [threading.Thread(target=go, args=(i,)) for i in range(len(ranges))]
        for t in ts:
            t.start()
        for t in ts:
            t.join()
    tot = {k: sum(a[k] for a in acc) for k in acc[0]}
    return dict(dx=dx, ddelta=ddelta, dA=tot["dA"], dB=tot["dB"], dC=tot["dC"], dh0=dh0,
                dD=tot["dD"] if D is not None else None,
                ddelta_bias=tot["dbias"] if delta_bias is not None else None, dz=dz)


def causal_conv1d(x, weight, bias=None, state=None, silu=True, threads: int = 1, lib=None):
    """Causal depthwise conv1d (+ SiLU) of ssm_oracle.c.  x: (Bt, T, Dd);
    weight: (Dd, K); bias: (Dd,); state: (Bt, Dd, K-1) inputs before the
    sequence (oldest first) or None.  Returns (out (Bt,T,Dd), state_out
    (Bt,Dd,K-1)) in fp64."""
    lib = lib or load()
    x, weight, bias, state = _f64(x), _f64(weight), _f64(bias), _f64(state)
    Bt, T, Dd = x.shape
    K = weight.shape[1]
    assert weight.shape == (Dd, K) and K >= 1
    assert bias is None or bias.shape == (Dd,)
    assert state is None or state.shape == (Bt, Dd, K - 1)
    out = np.zeros((Bt, T, Dd))
    st_out = np.zeros((Bt, Dd, K - 1))

    def go(c0, c1):
        lib.oracle_causal_conv1d(_ptr(x), _ptr(weight), _ptr(bias), _ptr(state), _ptr(out),
                                 _ptr(st_out), int(bool(silu)), Bt, T, Dd, K, c0, c1)

    _run_chains(go, Bt * Dd, threads)
    return out, st_out


def conv1d_update(state, x, weight, bias=None, silu=True, lib=None):
    """One decode token.  state: (Bt, Dd, K-1) (not modified: the new state is
    returned); x: (Bt, Dd).  Returns (out (Bt, Dd), new_state)."""
    lib = lib or load()
    st = _f64(state).copy()
    x, weight, bias = _f64(x), _f64(weight), _f64(bias)
    Bt, Dd = x.shape
    K = weight.shape[1]
    assert st.shape == (Bt, Dd, K - 1)
    out = np.zeros((Bt, Dd))
    lib.oracle_conv1d_update(_ptr(st), _ptr(x), _ptr(weight), _ptr(bias), _ptr(out),
                             int(bool(silu)), Bt, Dd, K, 0, Bt * Dd)
    return out, st


def sequence_order(height: int, width: int, direction: int):
    """The order in which the 2-D scans of the youngju.dev guide's VMamba
    section (section 9, image processing) visit the height x width patches:
    0 row-major (left to right, top to bottom), 1 its reverse, 2 column-major
    (the patch grid transposed), 3 its reverse.  Returns perm with
    perm[s] = the row-major index of the patch at scan step s."""
    idx = np.arange(height * width).reshape(height, width)
    seq = idx.reshape(-1) if direction in (0, 1) else idx.T.reshape(-1)
    return seq[::-1].copy() if direction in (1, 3) else seq


def scan_2d(x, delta, A, B, C, height, width, direction, D=None, z=None, delta_bias=None,
            delta_softplus=True, h0=None, threads: int = 1, lib=None):
    """One direction of the 2-D scan: the sequence (row-major patches, axis 1)
    is visited in `sequence_order`, scanned, and y is returned at each patch's
    own (row-major) position; last_state is the state after the last visited
    patch."""
    perm = sequence_order(height, width, direction)
    pick = lambda a: None if a is None else np.ascontiguousarray(np.asarray(a)[:, perm])
    y, last = selective_scan(pick(x), pick(delta), A, pick(B), pick(C), D=D, z=pick(z),
                             delta_bias=delta_bias, delta_softplus=delta_softplus, h0=h0,
                             threads=threads, lib=lib)
    out = np.empty_like(y)
    out[:, perm] = y
    return out, last


def ssd_scan(x, dt, A, B, C, D=None, z=None, dt_bias=None, dt_softplus=True, h0=None,
             threads: int = 1, lib=None):
    """The Mamba-2 multi-head scan, step by step in fp64 (oracle_ssd_scan).
    x, z: (Bt, T, H, P); dt: (Bt, T, H); A, D, dt_bias: (H,); B, C: (Bt, T, N);
    h0: (Bt, H, P, N).  Returns (y (Bt, T, H, P), last_state (Bt, H, P, N))."""
    lib = lib or load()
    x, dt, A, B, C = _f64(x), _f64(dt), _f64(A), _f64(B), _f64(C)
    D, z, dt_bias, h0 = _f64(D), _f64(z), _f64(dt_bias), _f64(h0)
    Bt, T, H, P = x.shape
    N = B.shape[2]
    assert dt.shape == (Bt, T, H) and A.shape == (H,)
    assert B.shape == (Bt, T, N) and C.shape == (Bt, T, N)
    assert z is None or z.shape == x.shape
    assert h0 is None or h0.shape == (Bt, H, P, N)
    y = np.zeros((Bt, T, H, P), dtype=np.float64)
    last = np.zeros((Bt, H, P, N), dtype=np.float64)

    def go(c0, c1):
        lib.oracle_ssd_scan(_ptr(x), _ptr(dt), _ptr(dt_bias), int(bool(dt_softplus)), _ptr(A),
                            _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(h0), _ptr(y), _ptr(last),
                            Bt, T, H, P, N, c0, c1)

    _run_chains(go, Bt * H * P, threads)
    return y, last


def dt_proj(xdt, W, threads: int = 1, lib=None):
    """delta = xdt[:, :rank] @ W.T, row by row in fp64 (oracle_dt_proj).
    xdt: (M, ldx) with ldx >= rank; only its first rank = W.shape[1] columns
    are read.  W: (D, rank).  Returns (M, D)."""
    lib = lib or load()
    xdt, W = _f64(xdt), _f64(W)
    M, ldx = xdt.shape
    D, rank = W.shape
    assert ldx >= rank
    out = np.zeros((M, D), dtype=np.float64)

    def go(r0, r1):
        lib.oracle_dt_proj(_ptr(xdt), ldx, _ptr(W), _ptr(out), M, rank, D, r0, r1)

    _run_chains(go, M, threads)
    return out
