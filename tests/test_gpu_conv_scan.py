"""GPU parity of the fused prologue + scan (ssm_conv_scan_fwd, through the C
ABI) against the oracle's causal conv1d + SiLU followed by its selective scan,
on the same seeded inputs.  The oracle's filtered x is fp64 and unrounded, as
the kernel's stays fp32 in registers.  Tolerances as for the scan: 1e-5 fp32,
2e-2 bf16 io with fp32 state (gpu_util.err)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import gpu_util as G
import oracle
from selective_scan_ssm_amd import inputs as gen

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from selective_scan_ssm_amd import _lib
    _lib.load()


def run(inp, cp, softplus=True, tag=""):
    from selective_scan_ssm_amd import ops
    io = inp["io"]
    Bt, T, Dd, N = inp["batch"], inp["seqlen"], inp["d_inner"], inp["d_state"]
    K = cp["conv_w"].shape[1]
    G.say(f"[conv-scan] {tag} B={Bt} T={T} D={Dd} N={N} K={K} io={io} "
          f"window={cp['conv_state'] is not None} bias={cp['conv_b'] is not None}")
    t = G.device_inputs(inp)
    y, last, win = ops.conv_scan_fwd(t["x"], G.to_torch(cp["conv_w"], gen.F32), t["delta"], t["A"], t["B"],
                                     t["C"], conv_bias=G.to_torch(cp["conv_b"], gen.F32),
                                     conv_state=G.to_torch(cp["conv_state"], io), D=t["D"], z=t["z"],
                                     delta_bias=t["delta_bias"], delta_softplus=softplus, h0=t["h0"],
                                     return_last_state=True, return_conv_state=True)
    torch.cuda.synchronize()
    d = G.decoded(inp)
    st = None if cp["conv_state"] is None else gen.to_f64(cp["conv_state"], io)
    xc, wo = oracle.causal_conv1d(d["x"], cp["conv_w"], cp["conv_b"], st, silu=True, threads=G.ORACLE_THREADS)
    yo, lo = oracle.selective_scan(xc, d["delta"], d["A"], d["B"], d["C"], D=d["D"], z=d["z"],
                                   delta_bias=d["delta_bias"], delta_softplus=softplus, h0=d["h0"],
                                   threads=G.ORACLE_THREADS)
    ey, el = G.err(G.from_torch(y), yo), G.err(G.from_torch(last), lo)
    tol = G.TOL[io]
    if io == gen.F32:
        # bounded by what fp32 arithmetic itself loses on this input (the
        # filtered x rounded to fp32, then the scan evaluated in fp32)
        tol, e32 = G.fp32_tolerance(yo, lo, x=xc, delta=d["delta"], A=d["A"], B=d["B"], C=d["C"], D=d["D"],
                                    z=d["z"], delta_bias=d["delta_bias"], softplus=softplus, h0=d["h0"])
        G.say(f"[conv-scan] {tag} plain fp32 evaluation err={e32:.3e}")
    del xc
    G.say(f"[conv-scan] {tag} err_y={ey:.3e} err_last={el:.3e} tol={tol:g}")
    assert ey <= tol and el <= tol, (ey, el)
    # the window after the sequence is a copy of inputs: bit-exact
    assert np.array_equal(G.from_torch(win), wo)


def test_mamba2p8b_layer_full_launch():
    # the benchmark's launch: 4 x 8192 x 5120, d_state 16, bf16, width 4 --
    # every output and final state against the oracle
    inp = gen.workload_inputs(3)
    cp = gen.make_conv_params(4, 5120, 4, io=gen.BF16, seed=31)
    run(inp, cp, tag="2.8b")


@pytest.mark.parametrize("io", [gen.BF16, gen.F32])
@pytest.mark.parametrize("K", [1, 2, 3, 4])
def test_widths_with_window_segments_ragged(io, K):
    # 1000 channels (a partial tile and a partial wave), 2100 steps (four
    # segments: the conv reads three rows of the previous segment), a window
    # before step 0 and h0
    inp = gen.make_inputs(2, 2100, 1000, 16, io=io, h0_kind="normal", seed=600 + K)
    cp = gen.make_conv_params(2, 1000, K, io=io, seed=610 + K, with_state=True)
    run(inp, cp, tag=f"K{K}")


@pytest.mark.parametrize("T", [1, 2, 3, 5, 16, 17, 33, 40])
def test_short_sequences(T):
    # sequences inside the first blocks, where the window substitutes the
    # rows before step 0
    inp = gen.make_inputs(3, T, 130, 16, io=gen.BF16, h0_kind="normal", seed=620 + T)
    cp = gen.make_conv_params(3, 130, 4, io=gen.BF16, seed=630 + T, with_state=True)
    run(inp, cp, tag=f"T{T}")


def test_no_bias_no_window_no_gate():
    inp = gen.make_inputs(2, 700, 256, 16, io=gen.F32, seed=640, with_z=False, with_D=False)
    cp = gen.make_conv_params(2, 256, 4, io=gen.F32, seed=641, with_bias=False)
    run(inp, cp, tag="plain")


@pytest.mark.parametrize("N", [1, 4, 8])
def test_other_state_sizes(N):
    # below d_state 16 the filtered x goes through the workspace
    inp = gen.make_inputs(2, 300, 200, N, io=gen.BF16, a_kind="sm1", h0_kind="normal", seed=650 + N)
    cp = gen.make_conv_params(2, 200, 4, io=gen.BF16, seed=660 + N, with_state=True)
    run(inp, cp, tag=f"N{N}")


def test_two_workgroups_per_cu():
    # 1280 tiles: two persistent workgroups per CU
    inp = gen.make_inputs(16, 1200, 5120, 16, io=gen.BF16, seed=670)
    cp = gen.make_conv_params(16, 5120, 4, io=gen.BF16, seed=671, with_state=True)
    run(inp, cp, tag="two-per-cu")


def test_empty_sequence():
    from selective_scan_ssm_amd import ops
    inp = gen.make_inputs(2, 0, 70, 16, io=gen.BF16, h0_kind="normal", seed=680)
    cp = gen.make_conv_params(2, 70, 4, io=gen.BF16, seed=681, with_state=True)
    t = G.device_inputs(inp)
    st = G.to_torch(cp["conv_state"], gen.BF16)
    y, last, win = ops.conv_scan_fwd(t["x"], G.to_torch(cp["conv_w"], gen.F32), t["delta"], t["A"], t["B"],
                                     t["C"], conv_state=st, D=t["D"], z=t["z"], delta_bias=t["delta_bias"],
                                     h0=t["h0"], return_last_state=True, return_conv_state=True)
    torch.cuda.synchronize()
    assert torch.equal(last, t["h0"])
    assert torch.equal(win.view(torch.int16), st.view(torch.int16))
