"""The entry points under HIP graph capture (torch.cuda.CUDAGraph on ROCm):
one call captured, then replayed three times with new inputs copied in
eagerly between replays; every replay must equal an eager call on the same
inputs bit for bit (the kernels are deterministic).  The scan kernels clear
their scratch with a kernel, not a memset, so nothing in a captured call
depends on a memset node."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import gpu_util as G
from selective_scan_ssm_amd import inputs as gen

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from selective_scan_ssm_amd import _lib
    _lib.load()


def replay_matches_eager(static, fn, refill, reps=3):
    """Capture fn(static) once, then for each replay refill the inputs
    eagerly, replay, and compare with an eager call on the same inputs."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):                 # warm up outside the capture
        fn(static)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = fn(static)
    for r in range(reps):
        refill(static, r)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = fn(static)
        torch.cuda.synchronize()
        outs = out if isinstance(out, (tuple, list)) else (out,)
        refs = ref if isinstance(ref, (tuple, list)) else (ref,)
        for a, b in zip(outs, refs):
            assert torch.equal(a, b), f"replay {r} differs from the eager call"
        G.say(f"[graph] replay {r} equals the eager call")


def test_graph_scan_fwd_rows_kernel():
    from selective_scan_ssm_amd import ops
    # d_state 16 with segments: the persistent row kernel, its ticket and hand-off words
    inp = gen.make_inputs(2, 1100, 320, 16, io=gen.BF16, h0_kind="normal", seed=60)
    st = G.device_inputs(inp)

    def fn(t):
        return ops.scan_fwd(t["x"], t["delta"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"],
                            delta_bias=t["delta_bias"], h0=t["h0"], return_last_state=True)

    def refill(t, r):
        t["x"].copy_(torch.randn(t["x"].shape, device="cuda").to(t["x"].dtype))
        t["h0"].copy_(torch.randn(t["h0"].shape, device="cuda"))
    replay_matches_eager(st, fn, refill)


def test_graph_ssd_and_prologue():
    from selective_scan_ssm_amd import ops
    si = gen.make_ssd_inputs(2, 150, 3, 32, 64, io=gen.BF16, h0_kind="normal", seed=61)
    st = {k: G.to_torch(si[k], gen.BF16) for k in ("x", "dt", "z", "B", "C")}
    st.update({k: G.to_torch(si[k], gen.F32) for k in ("A", "D", "dt_bias", "h0")})
    pi = gen.make_dtproj_inputs(300, 48, 136, 80, io=gen.BF16, seed=62)
    st["x_dbl"], st["W"] = G.to_torch(pi["x_dbl"], gen.BF16), G.to_torch(pi["W"], gen.BF16)
    st["cx"] = torch.randn(2, 90, 136, device="cuda").to(torch.bfloat16)
    st["cw"] = torch.randn(136, 4, device="cuda") * 0.5

    def fn(t):
        y, last = ops.ssd_scan_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"],
                                   dt_bias=t["dt_bias"], h0=t["h0"], return_last_state=True)
        dl = ops.dt_proj(t["x_dbl"][:, :48], t["W"])
        cv = ops.causal_conv1d(t["cx"], t["cw"], None, silu=True)
        return y, last, dl, cv

    def refill(t, r):
        for k in ("x", "x_dbl", "cx"):
            t[k].copy_(torch.randn(t[k].shape, device="cuda").to(t[k].dtype))
    replay_matches_eager(st, fn, refill)


def test_graph_backward_with_checkpoints():
    from selective_scan_ssm_amd import ops
    inp = gen.make_inputs(2, 200, 128, 16, io=gen.BF16, h0_kind="normal", seed=63)
    st = G.device_inputs(inp)
    st["dout"] = torch.randn(st["x"].shape, device="cuda").to(torch.bfloat16)
    st["ck"] = torch.empty(ops.ckpt_shape(2, 200, 128, 16), dtype=torch.float32, device="cuda")
    kw = lambda t: dict(D=t["D"], z=t["z"], delta_bias=t["delta_bias"], h0=t["h0"])

    def fn(t):
        y = ops.scan_fwd(t["x"], t["delta"], t["A"], t["B"], t["C"], ckpt_out=t["ck"], **kw(t))
        g = ops.scan_bwd(t["x"], t["delta"], t["A"], t["B"], t["C"], t["dout"], ckpt=t["ck"], **kw(t))
        return [y] + [v for v in g.values() if v is not None]

    def refill(t, r):
        t["dout"].copy_(torch.randn(t["dout"].shape, device="cuda").to(torch.bfloat16))
        t["x"].copy_(torch.randn(t["x"].shape, device="cuda").to(torch.bfloat16))
    replay_matches_eager(st, fn, refill)


def test_graph_backward_self_contained():
    """ssm_scan_bwd computing its own checkpoints: its carry pass runs on the
    library's side stream, forked from and joined back into the captured
    stream; the captured call replays equal to eager calls."""
    from selective_scan_ssm_amd import ops
    inp = gen.make_inputs(2, 200, 128, 16, io=gen.BF16, h0_kind="normal", seed=64)
    st = G.device_inputs(inp)
    st["dout"] = torch.randn(st["x"].shape, device="cuda").to(torch.bfloat16)
    st["dlast"] = torch.randn(st["h0"].shape, device="cuda")

    def fn(t):
        g = ops.scan_bwd(t["x"], t["delta"], t["A"], t["B"], t["C"], t["dout"], D=t["D"], z=t["z"],
                         delta_bias=t["delta_bias"], h0=t["h0"], dlast=t["dlast"])
        return [v for v in g.values() if v is not None]

    def refill(t, r):
        t["dout"].copy_(torch.randn(t["dout"].shape, device="cuda").to(torch.bfloat16))
        t["delta"].copy_(torch.randn(t["delta"].shape, device="cuda").to(torch.bfloat16))
    replay_matches_eager(st, fn, refill)
