"""C ABI contract, checked on the CPU: the library loads, exports every entry
point the header declares, and rejects bad arguments before touching the HIP
runtime (so these calls never launch anything)."""
import ctypes
import os
import re

import pytest

from selective_scan_ssm_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("ssm_scan.h", "ssm_scan_testing.h")]
BENCH_HEADER = os.path.join(ROOT, "include", "ssm_bench.h")

OK, ENULL, ESHAPE, EDTYPE, EALIGN, EWS, EHIP, EALIAS, EWAIT = 0, -1, -2, -3, -4, -5, -6, -7, -8
F32, BF16 = 0, 1
MB = 1 << 20


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from selective_scan_ssm_amd import build
        build.build()
    return _lib.load()


def header_functions(paths=HEADERS):
    out = set()
    for path in paths:
        src = open(path).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        out |= set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", src, re.M))
    return sorted(out)


def test_header_declares_the_boundary():
    fns = header_functions()
    assert set(fns) == set(_lib.EXPORTS), fns
    assert set(header_functions([BENCH_HEADER])) == set(_lib.BENCH_EXPORTS)
    # the measurement helpers are not part of the scan library's ABI
    assert not set(_lib.BENCH_EXPORTS) & set(fns)


def test_exports_every_declared_symbol(lib):
    for name in header_functions():
        assert hasattr(lib, name), name
    assert lib.ssm_abi_version() == _lib.ABI_VERSION == 3
    for name in _lib.BENCH_EXPORTS:
        assert not hasattr(lib, name), name


@pytest.fixture(scope="module")
def bench_lib():
    if not os.path.exists(_lib.BENCH_LIB_PATH):
        from selective_scan_ssm_amd import build
        build.build()
    return _lib.load_bench()


def test_bench_library_exports(bench_lib):
    for name in header_functions([BENCH_HEADER]):
        assert hasattr(bench_lib, name), name


def test_status_strings(lib):
    for code in (OK, ENULL, ESHAPE, EDTYPE, EALIGN, EWS, EHIP, EALIAS, EWAIT):
        s = lib.ssm_status_string(code).decode()
        assert s.startswith("SSM_"), s
    assert "unknown" in lib.ssm_status_string(12345).decode()


class FakeDev:
    """Distinct, well-aligned fake device addresses: never dereferenced
    because every call below fails validation (or is a documented no-op)."""

    def __init__(self):
        self.base = 0x7f0000000000
        self.off = 0

    def __call__(self, nbytes=64 * MB):
        p = self.base + self.off
        self.off += (nbytes + 4095) & ~4095
        return p


def scan_args(batch=2, seqlen=16, dim=8, dstate=4, io=F32, **over):
    f = FakeDev()
    a = dict(x=f(), delta=f(), delta_bias=f(), softplus=1, A=f(), B=f(), C=f(), D=f(), z=f(),
             h0=f(), y=f(), last=f(), batch=batch, seqlen=seqlen, dim=dim, dstate=dstate, io=io,
             ws=f(), ws_bytes=64 * MB, stream=None)
    a.update(over)
    return a


def call_scan(lib, a):
    return lib.ssm_scan_fwd(a["x"], a["delta"], a["delta_bias"], a["softplus"], a["A"], a["B"],
                            a["C"], a["D"], a["z"], a["h0"], a["y"], a["last"], a["batch"],
                            a["seqlen"], a["dim"], a["dstate"], a["io"], a["ws"], a["ws_bytes"],
                            a["stream"])


@pytest.mark.parametrize("over,code", [
    (dict(x=None), ENULL), (dict(delta=None), ENULL), (dict(A=None), ENULL),
    (dict(B=None), ENULL), (dict(C=None), ENULL), (dict(y=None), ENULL),
    (dict(dstate=0), ESHAPE), (dict(dstate=17), ESHAPE), (dict(batch=-1), ESHAPE),
    (dict(seqlen=-3), ESHAPE), (dict(dim=-1), ESHAPE), (dict(batch=70000), ESHAPE),
    (dict(batch=1 << 40, seqlen=1 << 40), ESHAPE),
    (dict(io=2), EDTYPE), (dict(io=-1), EDTYPE),
    (dict(x=0x7f0000000002), EALIGN), (dict(io=BF16, x=0x7f0000000001), EALIGN),
    (dict(A=0x7f0000000002), EALIGN), (dict(h0=0x7f000000000e), EALIGN),
    (dict(io=BF16, ws=None, ws_bytes=0), EWS), (dict(io=BF16, ws_bytes=16), EWS),
    (dict(ws=None, ws_bytes=0), EWS), (dict(dim=1 << 40, seqlen=1), ESHAPE),
])
def test_scan_validation(lib, over, code):
    assert call_scan(lib, scan_args(**over)) == code


def test_scan_alias_detection(lib):
    a = scan_args()
    a["y"] = a["x"] + 64           # inside x
    assert call_scan(lib, a) == EALIAS
    a = scan_args()
    a["last"] = a["h0"]            # last_state may not alias h0
    assert call_scan(lib, a) == EALIAS
    a = scan_args()
    a["y"] = a["last"]
    assert call_scan(lib, a) == EALIAS


def test_scan_empty_is_noop(lib):
    # batch == 0 or d_inner == 0: nothing to read or write; returns before any launch
    assert call_scan(lib, scan_args(batch=0)) == OK
    assert call_scan(lib, scan_args(dim=0)) == OK
    assert call_scan(lib, scan_args(batch=0, x=None, delta=None, y=None)) == OK


def test_sm1_workspace(lib):
    # the tiled SM1 kernel keeps every carry inside one workgroup: no workspace
    assert lib.sm1_scan_workspace_bytes(8, 4096, 1536, F32) == 0
    assert lib.sm1_scan_workspace_bytes(2, 16, 8, BF16) == 0
    # d_inner too wide for its 32-bit round offsets: handed to the general kernel
    need = lib.sm1_scan_workspace_bytes(1, 1, 1 << 22, F32)
    assert need > 0
    assert call_sm1(lib, scan_args(batch=1, seqlen=1, dstate=1, dim=1 << 22, ws=None, ws_bytes=0)) == EWS


def test_workspace_sizes(lib):
    assert lib.ssm_scan_workspace_bytes(2, 0, 8, 4, F32) == 0            # nothing to launch
    assert lib.ssm_scan_workspace_bytes(2, 16, 8, 4, F32) > 0             # ticket + carried states
    assert lib.ssm_scan_workspace_bytes(4, 8192, 5120, 16, BF16) < (64 << 20)
    assert lib.ssm_scan_workspace_bytes(2, 16, 8, 0, F32) == (1 << 64) - 1
    assert lib.ssm_scan_workspace_bytes(2, 16, 8, 4, 7) == (1 << 64) - 1
    assert lib.sm1_scan_workspace_bytes(2, 16, 8, 9) == (1 << 64) - 1
    assert lib.sm1_scan_workspace_bytes(8, 4096, 1536, F32) < (1 << 40)


def call_sm1(lib, a):
    return lib.sm1_scan_fwd(a["x"], a["delta"], a["delta_bias"], a["softplus"], a["A"], a["B"],
                            a["C"], a["D"], a["z"], a["h0"], a["y"], a["last"], a["batch"],
                            a["seqlen"], a["dim"], a["io"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("over,code", [
    (dict(x=None), ENULL), (dict(io=5), EDTYPE), (dict(batch=-2), ESHAPE),
    (dict(y=0x7f0000000003), EALIGN), (dict(batch=0), OK),
])
def test_sm1_validation(lib, over, code):
    assert call_sm1(lib, scan_args(dstate=1, **over)) == code


def call_step(lib, a):
    return lib.ssm_state_update(a["h0"], a["x"], a["delta"], a["delta_bias"], a["softplus"], a["A"],
                                a["B"], a["C"], a["D"], a["z"], a["y"], a["batch"], a["dim"],
                                a["dstate"], a["io"], a["stream"])


@pytest.mark.parametrize("over,code", [
    (dict(h0=None), ENULL), (dict(x=None), ENULL), (dict(y=None), ENULL),
    (dict(dstate=17), ESHAPE), (dict(dstate=0), ESHAPE), (dict(io=3), EDTYPE),
    (dict(h0=0x7f0000000002), EALIGN), (dict(batch=0), OK), (dict(dim=0), OK),
    # grid of one lane quad per chain, 64 chains per workgroup: below 2^32 lanes
    (dict(batch=1 << 16, dim=1 << 14), ESHAPE), (dict(batch=1, dim=1 << 30), ESHAPE),
])
def test_state_update_validation(lib, over, code):
    assert call_step(lib, scan_args(**over)) == code


def test_state_update_alias(lib):
    a = scan_args()
    a["y"] = a["x"]
    assert call_step(lib, a) == EALIAS


# ------------------------------------------------------------------ backward
def bwd_args(batch=2, seqlen=16, dim=8, dstate=4, io=F32, **over):
    f = FakeDev()
    a = dict(x=f(), delta=f(), delta_bias=f(), softplus=1, A=f(), B=f(), C=f(), D=f(), z=f(),
             h0=f(), dout=f(), dlast=f(), dx=f(), ddelta=f(), ddelta_bias=f(), dA=f(), dB=f(),
             dC=f(), dD=f(), dz=f(), dh0=f(), batch=batch, seqlen=seqlen, dim=dim, dstate=dstate,
             io=io, ws=f(), ws_bytes=16, stream=None)   # workspace too small: never launches
    a.update(over)
    return a


def call_bwd(lib, a):
    return lib.ssm_scan_bwd(a["x"], a["delta"], a["delta_bias"], a["softplus"], a["A"], a["B"],
                            a["C"], a["D"], a["z"], a["h0"], a["dout"], a["dlast"], a["dx"],
                            a["ddelta"], a["ddelta_bias"], a["dA"], a["dB"], a["dC"], a["dD"],
                            a["dz"], a["dh0"], a["batch"], a["seqlen"], a["dim"], a["dstate"],
                            a["io"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("over,code", [
    (dict(), EWS), (dict(ws=None, ws_bytes=0), EWS),
    (dict(x=None), ENULL), (dict(dout=None), ENULL), (dict(dx=None), ENULL),
    (dict(ddelta=None), ENULL), (dict(dA=None), ENULL), (dict(dB=None), ENULL),
    (dict(dC=None), ENULL), (dict(dz=None), ENULL), (dict(A=None), ENULL),
    (dict(dstate=0), ESHAPE), (dict(dstate=17), ESHAPE), (dict(batch=-1), ESHAPE),
    (dict(seqlen=-1), ESHAPE), (dict(batch=70000), ESHAPE),
    # one batch row of x must span less than 2 GiB (32-bit offsets)
    (dict(seqlen=1 << 16, dim=1 << 14), ESHAPE), (dict(seqlen=1 << 27, dstate=16), ESHAPE),
    (dict(io=2), EDTYPE),
    (dict(dx=0x7f0000000002), EALIGN), (dict(io=BF16, dB=0x7f0000000001), EALIGN),
    (dict(dA=0x7f0000000002), EALIGN), (dict(dlast=0x7f0000000006), EALIGN),
])
def test_bwd_validation(lib, over, code):
    assert call_bwd(lib, bwd_args(**over)) == code


def test_bwd_optional_outputs(lib):
    # without z, dz may be NULL; dD, ddelta_bias, dh0 and dlast are optional
    a = bwd_args(z=None, dz=None, dD=None, ddelta_bias=None, dh0=None, dlast=None)
    assert call_bwd(lib, a) == EWS          # valid up to the (too small) workspace


def test_bwd_alias_detection(lib):
    a = bwd_args()
    a["dx"] = a["x"] + 64
    assert call_bwd(lib, a) == EALIAS
    a = bwd_args()
    a["dB"] = a["dC"]
    assert call_bwd(lib, a) == EALIAS
    a = bwd_args()
    a["dh0"] = a["dlast"]
    assert call_bwd(lib, a) == EALIAS


def test_bwd_workspace_sizes(lib):
    # checkpoints every 16 steps + per-tile partials of dB, dC + per-(row,
    # segment) partials of dA, dD, dbias and the segment carries (glocal,
    # sum of Delta): the sweep cuts each sequence into 8 segments at this shape
    need = lib.ssm_scan_bwd_workspace_bytes(4, 8192, 5120, 16, BF16)
    ckpt = 4 * 512 * 5120 * 16 * 4
    parts = 2 * 80 * 4 * 8192 * 16 * 4
    segs = 4 * 8 * 5120 * (2 * 16 + 3) * 4
    assert ckpt + parts + segs <= need < ckpt + parts + segs + (4 << 20)
    assert lib.ssm_scan_bwd_workspace_bytes(2, 16, 8, 0, F32) == (1 << 64) - 1
    assert lib.ssm_scan_bwd_workspace_bytes(2, 16, 8, 4, 9) == (1 << 64) - 1
    assert lib.ssm_scan_bwd_workspace_bytes(0, 0, 0, 4, F32) == 0


def bwd_segments(lib, batch, seqlen, dim, N, io):
    S, sblk = ctypes.c_int(-1), ctypes.c_int(-1)
    r = lib.ssm_testing_bwd_segments(batch, seqlen, dim, N, io, ctypes.byref(S), ctypes.byref(sblk))
    return r, S.value, sblk.value


def test_bwd_segments(lib):
    # the layer shapes: 80 x 4 and 24 x 8 (tile, batch row) sequences, 8
    # segments each (2560 and 1536 workgroups: whole rounds of 2 per CU)
    assert bwd_segments(lib, 4, 8192, 5120, 16, BF16) == (OK, 8, 64)
    assert bwd_segments(lib, 8, 2048, 1536, 16, BF16) == (OK, 8, 16)
    # one block, or nothing: one segment
    assert bwd_segments(lib, 2, 16, 70, 16, F32)[:2] == (OK, 1)
    assert bwd_segments(lib, 2, 0, 70, 16, F32)[:2] == (OK, 1)
    assert bwd_segments(lib, 0, 100, 70, 16, F32)[:2] == (OK, 1)
    # every split covers the blocks exactly once, at most 64 segments
    for shape in [(2, 100, 130, 4, F32), (1, 200_000, 5120, 16, BF16), (3, 1000, 96, 1, F32),
                  (2, 300, 200, 16, BF16), (1, 77, 70, 16, F32), (64, 4096, 5120, 16, BF16),
                  (1, 33, 1, 16, F32)]:
        r, S, sblk = bwd_segments(lib, *shape)
        nblk = (shape[1] + 15) // 16
        assert r == OK and 1 <= S <= 64 and (S - 1) * sblk < nblk <= S * sblk, (shape, S, sblk)
    assert bwd_segments(lib, 2, 16, 8, 0, F32)[0] == ESHAPE
    assert bwd_segments(lib, 2, 16, 8, 4, 7)[0] == EDTYPE
    assert lib.ssm_testing_bwd_segments(2, 16, 8, 4, F32, None, None) == ENULL


# ------------------------------------------------------- causal conv1d
def conv_args(batch=2, seqlen=16, dim=8, width=4, io=F32, **over):
    f = FakeDev()
    a = dict(x=f(), w=f(), bias=f(), st_in=f(), out=f(), st_out=f(), silu=1, batch=batch,
             seqlen=seqlen, dim=dim, width=width, io=io, stream=None)
    a.update(over)
    return a


def call_conv(lib, a):
    return lib.ssm_causal_conv1d_fwd(a["x"], a["w"], a["bias"], a["st_in"], a["out"], a["st_out"],
                                     a["silu"], a["batch"], a["seqlen"], a["dim"], a["width"],
                                     a["io"], a["stream"])


def call_conv_update(lib, a):
    return lib.ssm_causal_conv1d_update(a["st_in"], a["x"], a["w"], a["bias"], a["out"], a["silu"],
                                        a["batch"], a["dim"], a["width"], a["io"], a["stream"])


@pytest.mark.parametrize("over,code", [
    (dict(x=None), ENULL), (dict(out=None), ENULL), (dict(w=None), ENULL),
    (dict(width=0), ESHAPE), (dict(width=5), ESHAPE), (dict(batch=-1), ESHAPE),
    (dict(seqlen=-1), ESHAPE), (dict(batch=70000), ESHAPE), (dict(seqlen=1 << 20, dim=1 << 10), ESHAPE),
    (dict(io=4), EDTYPE), (dict(x=0x7f0000000002), EALIGN), (dict(io=BF16, out=0x7f0000000001), EALIGN),
    (dict(w=0x7f0000000002), EALIGN), (dict(batch=0), OK), (dict(dim=0), OK),
])
def test_conv_validation(lib, over, code):
    assert call_conv(lib, conv_args(**over)) == code


@pytest.mark.parametrize("over,code", [
    (dict(x=None), ENULL), (dict(st_in=None), ENULL), (dict(out=None), ENULL),
    (dict(width=9), ESHAPE), (dict(io=9), EDTYPE), (dict(st_in=0x7f0000000002), EALIGN),
    (dict(batch=0), OK),
])
def test_conv_update_validation(lib, over, code):
    assert call_conv_update(lib, conv_args(**over)) == code


def test_conv_alias(lib):
    a = conv_args()
    a["out"] = a["x"]
    assert call_conv(lib, a) == EALIAS
    a = conv_args()
    a["st_out"] = a["st_in"]
    assert call_conv(lib, a) == EALIAS
    a = conv_args()
    a["out"] = a["st_in"]
    assert call_conv_update(lib, a) == EALIAS


# ------------------------------------------------------------- 2-D scan
def call_2d(lib, a, height=4, width=4, direction=1):
    return lib.ssm_scan_fwd_2d(a["x"], a["delta"], a["delta_bias"], a["softplus"], a["A"], a["B"],
                               a["C"], a["D"], a["z"], a["h0"], a["y"], a["last"], a["batch"],
                               height, width, a["dim"], a["dstate"], direction, a["io"], a["ws"],
                               a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("over,kw,code", [
    (dict(), dict(direction=4), ESHAPE), (dict(), dict(direction=-1), ESHAPE),
    (dict(), dict(height=-1), ESHAPE), (dict(), dict(height=1 << 40, width=1 << 40), ESHAPE),
    (dict(x=None), dict(), ENULL), (dict(dstate=0), dict(), ESHAPE), (dict(io=3), dict(), EDTYPE),
    (dict(ws_bytes=16), dict(), EWS), (dict(ws=None, ws_bytes=0), dict(), EWS),
    (dict(batch=0), dict(), OK),
])
def test_scan_2d_validation(lib, over, kw, code):
    assert call_2d(lib, scan_args(**over), **kw) == code


def test_scan_2d_workspace(lib):
    fwd = lib.ssm_scan_workspace_bytes(2, 64, 96, 16, BF16)
    # d_state 16 visits every order in place: the forward's own workspace only
    for direction in range(4):
        assert lib.ssm_scan_2d_workspace_bytes(2, 8, 8, 96, 16, direction, 1, BF16) == fwd
    # other widths gather the column-major and reversed orders: a copy of x,
    # delta, z, B, C, y after the forward's workspace
    fwd8 = lib.ssm_scan_workspace_bytes(2, 64, 96, 8, BF16)
    assert lib.ssm_scan_2d_workspace_bytes(2, 8, 8, 96, 8, 0, 1, BF16) == fwd8
    for direction in (1, 2, 3):
        need = lib.ssm_scan_2d_workspace_bytes(2, 8, 8, 96, 8, direction, 1, BF16)
        assert need >= fwd8 + 2 * 64 * (4 * 96 + 2 * 8) * 2
    # a one-row grid visited column-major is the row-major order
    assert lib.ssm_scan_2d_workspace_bytes(2, 1, 64, 96, 8, 2, 1, BF16) == fwd8
    assert lib.ssm_scan_2d_workspace_bytes(2, 8, 8, 96, 0, 0, 1, BF16) == (1 << 64) - 1
    assert lib.ssm_scan_2d_workspace_bytes(2, 8, 8, 96, 16, 4, 1, BF16) == (1 << 64) - 1
    assert lib.ssm_scan_2d_workspace_bytes(2, 8, 8, 96, 16, -1, 1, BF16) == (1 << 64) - 1


def test_scan_status_validation(lib):
    # argument checks only (the query itself synchronises a stream)
    assert lib.ssm_scan_status(None, 4096, None) == ENULL
    assert lib.ssm_scan_status(FakeDev()(), 16, None) == EWS


def call_no_handoff(lib, a, spin):
    return lib.ssm_testing_scan_fwd_no_handoff(a["x"], a["delta"], a["delta_bias"], a["softplus"], a["A"],
                                               a["B"], a["C"], a["D"], a["z"], a["h0"], a["y"], a["last"],
                                               a["batch"], a["seqlen"], a["dim"], a["dstate"], a["io"],
                                               a["ws"], a["ws_bytes"], spin, a["stream"])


def test_no_handoff_hook_validation(lib):
    # the test hook validates exactly as ssm_scan_fwd, plus its poll bound
    assert call_no_handoff(lib, scan_args(dstate=16, ws_bytes=16), 64) == EWS
    assert call_no_handoff(lib, scan_args(dstate=16, ws_bytes=16), 0) == ESHAPE
    assert call_no_handoff(lib, scan_args(dstate=16, ws_bytes=16), 1 << 20) == ESHAPE
    assert call_no_handoff(lib, scan_args(x=None), 64) == ENULL
    assert call_no_handoff(lib, scan_args(batch=0), 64) == OK


# ------------------------------------------------------ Mamba-2 multi-head scan
def ssd_args(batch=2, seqlen=16, nheads=3, headdim=32, dstate=64, io=F32, **over):
    f = FakeDev()
    a = dict(x=f(), dt=f(), dt_bias=f(), softplus=1, A=f(), B=f(), C=f(), D=f(), z=f(), h0=f(), y=f(),
             last=f(), batch=batch, seqlen=seqlen, nheads=nheads, headdim=headdim, dstate=dstate, io=io,
             ws=f(), ws_bytes=64 * MB, stream=None)
    a.update(over)
    return a


def call_ssd(lib, a):
    return lib.ssd_scan_fwd(a["x"], a["dt"], a["dt_bias"], a["softplus"], a["A"], a["B"], a["C"], a["D"],
                            a["z"], a["h0"], a["y"], a["last"], a["batch"], a["seqlen"], a["nheads"],
                            a["headdim"], a["dstate"], a["io"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("over,code", [
    (dict(x=None), ENULL), (dict(dt=None), ENULL), (dict(A=None), ENULL), (dict(B=None), ENULL),
    (dict(C=None), ENULL), (dict(y=None), ENULL),
    (dict(dstate=16), ESHAPE), (dict(dstate=48), ESHAPE), (dict(dstate=128), ESHAPE),
    (dict(io=BF16, dstate=256), ESHAPE), (dict(headdim=24), ESHAPE), (dict(headdim=0), ESHAPE),
    (dict(batch=-1), ESHAPE), (dict(seqlen=-1), ESHAPE), (dict(nheads=-2), ESHAPE),
    (dict(seqlen=1 << 24, nheads=8, headdim=64), ESHAPE),      # one batch row past 2 GiB
    (dict(io=2), EDTYPE),
    (dict(x=0x7f0000000008), EALIGN), (dict(B=0x7f0000000004), EALIGN), (dict(h0=0x7f0000000008), EALIGN),
    (dict(A=0x7f0000000002), EALIGN), (dict(io=BF16, dt=0x7f0000000001), EALIGN),
    (dict(batch=0), OK), (dict(nheads=0), OK), (dict(batch=0, x=None, y=None), OK),
])
def test_ssd_validation(lib, over, code):
    assert call_ssd(lib, ssd_args(**over)) == code


def ssd_segments(lib, batch, seqlen, nheads, headdim, dstate, io):
    S, cps = ctypes.c_int(-1), ctypes.c_int(-1)
    r = lib.ssm_testing_ssd_segments(batch, seqlen, nheads, headdim, dstate, io, ctypes.byref(S),
                                     ctypes.byref(cps))
    return r, S.value, cps.value


def test_ssd_segments_and_workspace(lib):
    # the 2.7b layer (4 x 8 heads x 5 line tiles = 160 units, 128 chunks):
    # 8 segments of 16 chunks, 1280 workgroups (five rounds on 256 CUs); the
    # workspace holds 7 segment states per unit (8 waves x 2 tiles x 1 KB)
    # and 8 decay sums per unit
    assert ssd_segments(lib, 4, 8192, 8, 320, 64, BF16) == (OK, 8, 16)
    need = lib.ssd_scan_workspace_bytes(4, 8192, 8, 320, 64, BF16)
    state = 160 * 7 * 8 * 2 * 256 * 4
    assert need == state + ((160 * 8 * 4 + 255) & ~255)
    # the chunk kernel's shapes (fp32, or head size not a multiple of 64): no segments
    assert ssd_segments(lib, 8, 2048, 24, 96, 64, BF16)[:2] == (OK, 1)
    assert lib.ssd_scan_workspace_bytes(8, 2048, 24, 96, 64, BF16) == 0
    assert lib.ssd_scan_workspace_bytes(2, 300, 3, 64, 32, F32) == 0
    # plenty of units: one segment
    assert ssd_segments(lib, 64, 4096, 8, 320, 64, BF16)[:2] == (OK, 1)
    # every split covers the chunks once
    for shape in [(1, 1000, 2, 64, 32), (1, 4096, 1, 128, 64), (2, 65, 1, 64, 64), (1, 64, 1, 64, 32)]:
        r, S, cps = ssd_segments(lib, *shape, BF16)
        nch = (shape[1] + 63) // 64
        assert r == OK and 1 <= S <= 64 and (S - 1) * cps < nch <= S * cps, (shape, S, cps)
    assert lib.ssd_scan_workspace_bytes(2, 16, 3, 24, 64, F32) == (1 << 64) - 1
    assert lib.ssd_scan_workspace_bytes(2, 16, 3, 32, 64, 9) == (1 << 64) - 1
    assert ssd_segments(lib, 2, 16, 3, 24, 64, F32)[0] == ESHAPE
    assert lib.ssm_testing_ssd_segments(2, 16, 3, 32, 64, F32, None, None) == ENULL


def test_ssd_workspace_validation(lib):
    # a segmented shape: the workspace is required, 256-byte aligned and apart
    # from every tensor
    shape = dict(batch=1, seqlen=4096, nheads=1, headdim=128, dstate=64, io=BF16)
    need = lib.ssd_scan_workspace_bytes(1, 4096, 1, 128, 64, BF16)
    assert need > 0
    assert call_ssd(lib, ssd_args(**shape, ws=None, ws_bytes=0)) == EWS
    assert call_ssd(lib, ssd_args(**shape, ws_bytes=need - 1)) == EWS
    a = ssd_args(**shape)
    a["ws"] += 128
    assert call_ssd(lib, a) == EALIGN
    a = ssd_args(**shape)
    a["ws"] = a["x"]
    assert call_ssd(lib, a) == EALIAS
    # no workspace needed: NULL is fine
    assert call_ssd(lib, ssd_args(io=F32, ws=None, ws_bytes=0, batch=0)) == OK


def test_ssd_supported_shapes_pass_validation_rules(lib):
    # bf16 io also takes d_state 128; fp32 does not (its LDS staging would not fit)
    assert call_ssd(lib, ssd_args(io=BF16, dstate=128, batch=0)) == OK
    assert call_ssd(lib, ssd_args(io=F32, dstate=128, batch=0)) == ESHAPE


def test_ssd_alias_detection(lib):
    a = ssd_args()
    a["y"] = a["x"] + 64
    assert call_ssd(lib, a) == EALIAS
    a = ssd_args()
    a["last"] = a["h0"]
    assert call_ssd(lib, a) == EALIAS
    a = ssd_args()
    a["y"] = a["last"]
    assert call_ssd(lib, a) == EALIAS


# ------------------------------------------------------ measurement helpers
MB_ERR_ARG = -1


@pytest.mark.parametrize("args,code", [
    (dict(src=None), MB_ERR_ARG), (dict(bytes_=24), MB_ERR_ARG), (dict(src=0x7f0000000008), MB_ERR_ARG),
    (dict(dst="src+16"), MB_ERR_ARG), (dict(bytes_=0, src=None, dst=None), OK),
])
def test_mb_copy_validation(bench_lib, args, code):
    f = FakeDev()
    src, dst = f(), f()
    a = dict(src=src, dst=dst, bytes_=1 << 20)
    a.update(args)
    if a["dst"] == "src+16":
        a["dst"] = a["src"] + 16
    assert bench_lib.ssm_mb_copy(a["src"], a["dst"], a["bytes_"], None) == code


@pytest.mark.parametrize("op,blocks,iters,out,code", [
    (4, 1, 1, True, MB_ERR_ARG), (-1, 1, 1, True, MB_ERR_ARG), (0, -1, 1, True, MB_ERR_ARG),
    (0, 1, -1, True, MB_ERR_ARG), (0, 1, 1, False, MB_ERR_ARG), (3, 0, 1, False, OK),
])
def test_mb_valu_validation(bench_lib, op, blocks, iters, out, code):
    ptr = FakeDev()() if out else None
    assert bench_lib.ssm_mb_valu(op, ptr, blocks, iters, None) == code


# ------------------------------------------------------------------ dt_proj
def dtp_args(rows=256, rank=160, dim=512, ldx=192, io=BF16, **over):
    f = FakeDev()
    a = dict(xdt=f(), ldx=ldx, W=f(), out=f(), rows=rows, rank=rank, dim=dim, io=io, stream=None)
    a.update(over)
    return a


def call_dtp(lib, a):
    return lib.ssm_dt_proj(a["xdt"], a["ldx"], a["W"], a["out"], a["rows"], a["rank"], a["dim"], a["io"],
                           a["stream"])


@pytest.mark.parametrize("over,code", [
    (dict(xdt=None), ENULL), (dict(W=None), ENULL), (dict(out=None), ENULL),
    (dict(rank=0), ESHAPE), (dict(rank=-8), ESHAPE), (dict(rows=-1), ESHAPE), (dict(dim=-4), ESHAPE),
    (dict(rank=164), ESHAPE),                  # bf16 rank not a multiple of 8
    (dict(ldx=196), ESHAPE),                   # bf16 row stride not a multiple of 8
    (dict(ldx=152), ESHAPE),                   # row stride below the rank
    (dict(dim=510), ESHAPE),                   # d_inner not a multiple of 4
    (dict(io=F32, rank=162, ldx=192), ESHAPE),
    (dict(rows=1 << 62, ldx=1 << 8), ESHAPE),  # element count overflows
    (dict(io=5), EDTYPE),
    (dict(xdt=0x7f0000000008), EALIGN), (dict(W=0x7f0000000004), EALIGN), (dict(out=0x7f0000000002), EALIGN),
    (dict(rows=0), OK), (dict(dim=0), OK), (dict(rows=0, xdt=None, out=None), OK),
])
def test_dt_proj_validation(lib, over, code):
    assert call_dtp(lib, dtp_args(**over)) == code


def test_dt_proj_alias_detection(lib):
    a = dtp_args()
    a["out"] = a["xdt"] + 4096
    assert call_dtp(lib, a) == EALIAS
    a = dtp_args()
    a["out"] = a["W"]
    assert call_dtp(lib, a) == EALIAS


# ------------------------------------------------- checkpoints saved by the forward
def test_ckpt_bytes(lib):
    # batch x ceil(seqlen / 16) x d_inner x d_state fp32
    assert lib.ssm_scan_ckpt_bytes(2, 33, 8, 4) == 2 * 3 * 8 * 4 * 4
    assert lib.ssm_scan_ckpt_bytes(1, 0, 8, 16) == 0
    assert lib.ssm_scan_ckpt_bytes(1, 16, 8, 0) == (1 << 64) - 1
    assert lib.ssm_scan_ckpt_bytes(-1, 16, 8, 4) == (1 << 64) - 1


def call_fwd_ckpt(lib, a, ckpt):
    return lib.ssm_scan_fwd_ckpt(a["x"], a["delta"], a["delta_bias"], a["softplus"], a["A"], a["B"], a["C"],
                                 a["D"], a["z"], a["h0"], a["y"], a["last"], ckpt, a["batch"], a["seqlen"],
                                 a["dim"], a["dstate"], a["io"], a["ws"], a["ws_bytes"], a["stream"])


def test_fwd_ckpt_validation(lib):
    # d_state 16 always needs a workspace: a valid call stops at the 16-byte one
    base = dict(dstate=16, ws_bytes=16)
    a = scan_args(**base)
    ck = FakeDev().base + (1 << 36)
    assert call_fwd_ckpt(lib, a, ck) == EWS
    assert call_fwd_ckpt(lib, a, None) == ENULL
    assert call_fwd_ckpt(lib, a, ck + 8) == EALIGN
    assert call_fwd_ckpt(lib, a, a["y"]) == EALIAS
    assert call_fwd_ckpt(lib, a, a["h0"]) == EALIAS
    assert call_fwd_ckpt(lib, scan_args(batch=0, **base), None) == OK
    assert call_fwd_ckpt(lib, scan_args(dstate=17, ws_bytes=16), ck) == ESHAPE


def call_bwd_ckpt(lib, a, ckpt):
    return lib.ssm_scan_bwd_ckpt(a["x"], a["delta"], a["delta_bias"], a["softplus"], a["A"], a["B"], a["C"],
                                 a["D"], a["z"], a["h0"], a["dout"], a["dlast"], ckpt, a["dx"], a["ddelta"],
                                 a["ddelta_bias"], a["dA"], a["dB"], a["dC"], a["dD"], a["dz"], a["dh0"],
                                 a["batch"], a["seqlen"], a["dim"], a["dstate"], a["io"], a["ws"],
                                 a["ws_bytes"], a["stream"])


def test_bwd_ckpt_validation(lib):
    a = bwd_args()
    ck = FakeDev().base + (1 << 36)
    assert call_bwd_ckpt(lib, a, ck) == EWS              # valid up to the (too small) workspace
    assert call_bwd_ckpt(lib, a, None) == ENULL
    assert call_bwd_ckpt(lib, a, ck + 4) == EALIGN
    assert call_bwd_ckpt(lib, a, a["dx"]) == EALIAS      # an output over the checkpoints
    assert call_bwd_ckpt(lib, a, a["dh0"]) == EALIAS


# ------------------------------------------------- the allocation-free forward
def call_noalloc(lib, a):
    return lib.ssm_scan_fwd_noalloc(a["x"], a["delta"], a["delta_bias"], a["softplus"], a["A"], a["B"],
                                    a["C"], a["D"], a["z"], a["h0"], a["y"], a["last"], a["batch"],
                                    a["seqlen"], a["dim"], a["dstate"], a["io"], a["stream"])


def test_noalloc_scratch_limit(lib):
    # 512 bytes per state of a 64-channel tile, after a 256-byte header and the
    # tiles' progress words: 2046 tiles at d_state 16 fit in 16 MiB, 2048 do not
    fits = lib.ssm_scan_workspace_bytes(2, 4096, 2046 * 32, 16, BF16)
    assert 0 < fits <= _lib.SSM_SCRATCH_BYTES
    assert lib.ssm_scan_workspace_bytes(32, 4096, 4096, 16, BF16) > _lib.SSM_SCRATCH_BYTES
    f = FakeDev()
    big = dict((k, f(1 << 32)) for k in ("x", "delta", "delta_bias", "A", "B", "C", "D", "z", "h0", "y", "last"))
    assert call_noalloc(lib, scan_args(batch=32, seqlen=4096, dim=4096, dstate=16, io=BF16, **big)) == -9
    assert "SCRATCH" in lib.ssm_status_string(-9).decode()


@pytest.mark.parametrize("over,code", [
    (dict(x=None), ENULL), (dict(dstate=0), ESHAPE), (dict(io=7), EDTYPE), (dict(A=0x7f0000000002), EALIGN),
    (dict(batch=0), OK), (dict(dim=0), OK),
])
def test_noalloc_validation(lib, over, code):
    assert call_noalloc(lib, scan_args(**over)) == code


def test_noalloc_alias_detection(lib):
    a = scan_args()
    a["y"] = a["x"]
    assert call_noalloc(lib, a) == EALIAS
