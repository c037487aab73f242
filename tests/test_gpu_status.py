"""The error path of the segment hand-off, forced from the host.

A forward scan cut into time segments hands each segment's final state to the
next through the workspace, and the successor's wait for it is bounded.  The
testing entry point ssm_testing_scan_fwd_no_handoff withholds every hand-off
and bounds the wait at a few polls, so every job past a tile's first segment
gives up while every kernel still ends normally.  The give-up must reach the
caller: ssm_scan_status reports SSM_ERR_WAIT, and the outputs that depend on a
given-up state are NaN.  A normal call on the same workspace then reports
SSM_OK again and matches the oracle."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import gpu_util as G
from selective_scan_ssm_amd import _lib, ops
from selective_scan_ssm_amd import inputs as gen

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _lib.load()


def _no_handoff(t, y, last, ws, shape, io, spin):
    lib = _lib.load()
    Bt, T, Dd, N = shape
    p = lambda a: None if a is None else a.data_ptr()
    return lib.ssm_testing_scan_fwd_no_handoff(
        p(t["x"]), p(t["delta"]), p(t["delta_bias"]), 1, p(t["A"]), p(t["B"]), p(t["C"]), p(t["D"]),
        p(t["z"]), p(t["h0"]), p(y), p(last), Bt, T, Dd, N, io, p(ws), ws.numel(), spin,
        torch.cuda.current_stream().cuda_stream)


# (batch, seqlen, d_inner, d_state, io, segment length in steps):
#   d_state 16 -- the row kernel, 2048 steps in 4 segments of 512;
#   d_state 4  -- the general kernel, 256 channel tiles (so it cuts segments),
#                 1024 steps in 2 segments of 512 (bf16 io: at 16.8M fp32
#                 outputs even a plain sequential fp32 evaluation strays past
#                 1e-5 somewhere, see the precision notes of the design)
@pytest.mark.parametrize("shape,io,seg", [((1, 2048, 128, 16), gen.BF16, 512),
                                          ((4, 1024, 4096, 4), gen.BF16, 512),
                                          ((1, 2048, 64, 16), gen.F32, 512)])
def test_forced_giveup_is_reported(shape, io, seg):
    Bt, T, Dd, N = shape
    G.say(f"[status] forced give-up B={Bt} T={T} D={Dd} N={N} io={io}")
    inp = gen.make_inputs(Bt, T, Dd, N, io=io, h0_kind="normal", seed=900 + N)
    t = G.device_inputs(inp)
    dt = t["x"].dtype
    need = ops.scan_workspace_bytes(Bt, T, Dd, N, dt)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    y = torch.empty_like(t["x"])
    last = torch.empty((Bt, Dd, N), dtype=torch.float32, device="cuda")
    io_code = _lib.SSM_BF16 if io == gen.BF16 else _lib.SSM_F32
    rc = _no_handoff(t, y, last, ws, shape, io_code, 64)
    assert rc == 0, _lib.status_string(rc)
    st = ops.scan_status(ws)
    G.say(f"[status] after the forced give-up: {st} ({_lib.status_string(st)})")
    assert st == _lib.SSM_ERR_WAIT
    yg, lg = G.from_torch(y), G.from_torch(last)
    # the first segment of every tile never waits: its outputs are the normal call's
    yn, ln = ops.scan_fwd(t["x"], t["delta"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"],
                          delta_bias=t["delta_bias"], h0=t["h0"], return_last_state=True, workspace=ws)
    assert ops.scan_status(ws) == 0          # the next call clears the error word
    yn = G.from_torch(yn)
    assert np.array_equal(yg[:, :seg], yn[:, :seg])
    # every later step depends on a given-up state: NaN, never a plausible value
    assert np.all(np.isnan(yg[:, seg:]))
    assert np.all(np.isnan(lg))
    # and the normal call on the same workspace is right
    yo, lo = G.run_oracle(inp)
    tol = G.TOL[io]
    ey, el = G.err(yn, yo), G.err(G.from_torch(ln), lo)
    G.say(f"[status] normal call after it: err_y={ey:.3e} err_last={el:.3e}")
    assert ey <= tol and el <= tol


def test_status_ok_after_a_normal_call():
    inp = gen.make_inputs(2, 1500, 200, 16, io=gen.BF16, seed=905)
    t = G.device_inputs(inp)
    need = ops.scan_workspace_bytes(2, 1500, 200, 16, torch.bfloat16)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    ops.scan_fwd(t["x"], t["delta"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"],
                 delta_bias=t["delta_bias"], workspace=ws)
    assert ops.scan_status(ws) == 0
