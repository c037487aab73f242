"""ssm_scan_fwd_noalloc through the C ABI against ssm_scan_fwd (the existing
entry point, with a caller workspace) on the same inputs: two calls in a row,
the second with a smaller input, so the static scratch array is reused with
the first call's contents still in it.  Both entry points run the same
kernels, so the outputs must agree bit for bit."""
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


def noalloc(t, shape, io):
    lib = _lib.load()
    Bt, T, Dd, N = shape
    y = torch.empty_like(t["x"])
    last = torch.empty((Bt, Dd, N), dtype=torch.float32, device="cuda")
    p = lambda a: None if a is None else a.data_ptr()
    io_code = _lib.SSM_BF16 if io == gen.BF16 else _lib.SSM_F32
    rc = lib.ssm_scan_fwd_noalloc(p(t["x"]), p(t["delta"]), p(t["delta_bias"]), 1, p(t["A"]), p(t["B"]),
                                  p(t["C"]), p(t["D"]), p(t["z"]), p(t["h0"]), p(y), p(last), Bt, T, Dd, N,
                                  io_code, torch.cuda.current_stream().cuda_stream)
    assert rc == 0, _lib.status_string(rc)
    return y, last


def bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


@pytest.mark.parametrize("io", [gen.BF16, gen.F32])
def test_noalloc_matches_workspace_entry(io):
    # first: 4 batch rows x 1000 channels (64 tiles, the last partial) and 2100
    # steps (4 segments handed on through the scratch); second, smaller: 1 row
    # x 300 channels x 700 steps (one segment)
    for shape, seed in (((4, 2100, 1000, 16), 700), ((1, 700, 300, 16), 701)):
        Bt, T, Dd, N = shape
        G.say(f"[noalloc] B={Bt} T={T} D={Dd} N={N} io={io}")
        inp = gen.make_inputs(Bt, T, Dd, N, io=io, h0_kind="normal", seed=seed)
        t = G.device_inputs(inp)
        y, last = noalloc(t, shape, io)
        yr, lr = ops.scan_fwd(t["x"], t["delta"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"],
                              delta_bias=t["delta_bias"], h0=t["h0"], return_last_state=True)
        torch.cuda.synchronize()
        assert torch.equal(bits(y), bits(yr)), f"y differs at {shape}"
        assert torch.equal(bits(last), bits(lr)), f"last_state differs at {shape}"
        assert bool(torch.isfinite(last).all())


def test_noalloc_general_kernel_then_rows_kernel():
    # d_state 4 on 256 channel tiles (the general kernel, 2 segments), then a
    # smaller d_state-16 call: the scratch holds the first call's words
    for shape, seed in (((4, 1024, 4096, 4), 702), ((2, 600, 256, 16), 703)):
        Bt, T, Dd, N = shape
        G.say(f"[noalloc] B={Bt} T={T} D={Dd} N={N} bf16")
        inp = gen.make_inputs(Bt, T, Dd, N, io=gen.BF16, h0_kind="normal", seed=seed)
        t = G.device_inputs(inp)
        y, last = noalloc(t, shape, gen.BF16)
        yr, lr = ops.scan_fwd(t["x"], t["delta"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"],
                              delta_bias=t["delta_bias"], h0=t["h0"], return_last_state=True)
        torch.cuda.synchronize()
        assert torch.equal(bits(y), bits(yr)) and torch.equal(bits(last), bits(lr))
