"""GPU parity of the Mamba-2 multi-head scan (ssd_scan_fwd through the C ABI)
against the fp64 oracle (oracle_ssd_scan, pinned by the semiseparable-matrix
form and by the Mamba-1 scan with tied decays) on the same seeded inputs.

Tolerances as for the Mamba-1 scan (gpu_util.err, max relative error with an
rms floor): 1e-5 for fp32 io, 2e-2 for bf16 io.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import gpu_util as G
import oracle
from selective_scan_ssm_amd import inputs as gen

pytestmark = pytest.mark.gpu

IO = ("x", "dt", "z", "B", "C")
F32 = ("A", "D", "dt_bias", "h0")


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from selective_scan_ssm_amd import _lib
    _lib.load()
    assert len(_lib.hip_runtimes_mapped()) == 1


def run_gpu(inp, softplus=True):
    from selective_scan_ssm_amd import ops
    t = {k: G.to_torch(inp[k], inp["io"]) for k in IO}
    t.update({k: G.to_torch(inp[k], gen.F32) for k in F32})
    y, last = ops.ssd_scan_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"],
                               dt_bias=t["dt_bias"], dt_softplus=softplus, h0=t["h0"], return_last_state=True)
    torch.cuda.synchronize()
    return G.from_torch(y), G.from_torch(last)


def decoded(inp):
    d = {k: (None if inp[k] is None else gen.to_f64(inp[k], inp["io"])) for k in IO}
    d.update({k: (None if inp[k] is None else np.asarray(inp[k], np.float64)) for k in F32})
    return d


def run_oracle(inp, softplus=True, heads=None, chans=None):
    """The oracle on all chains, or on heads x channels (every batch row)."""
    d = decoded(inp)
    if heads is not None:
        hi, pi = np.asarray(heads), np.asarray(chans)
        sub = lambda a: None if a is None else np.ascontiguousarray(a[:, :, hi][:, :, :, pi])
        d = dict(d, x=sub(d["x"]), z=sub(d["z"]), dt=np.ascontiguousarray(d["dt"][:, :, hi]), A=d["A"][hi],
                 D=None if d["D"] is None else d["D"][hi],
                 dt_bias=None if d["dt_bias"] is None else d["dt_bias"][hi],
                 h0=None if d["h0"] is None else np.ascontiguousarray(d["h0"][:, hi][:, :, pi]))
    return oracle.ssd_scan(d["x"], d["dt"], d["A"], d["B"], d["C"], D=d["D"], z=d["z"], dt_bias=d["dt_bias"],
                           dt_softplus=softplus, h0=d["h0"], threads=G.ORACLE_THREADS)


def check(inp, softplus=True, tag=""):
    G.say(f"[ssd] {tag} B={inp['batch']} T={inp['seqlen']} H={inp['nheads']} P={inp['headdim']} "
          f"N={inp['d_state']} io={inp['io']}")
    y, last = run_gpu(inp, softplus)
    yo, lo = run_oracle(inp, softplus)
    ey, el = G.err(y, yo), G.err(last, lo)
    tol = G.TOL[inp["io"]]
    G.say(f"[ssd] {tag} err_y={ey:.2e} err_last={el:.2e} (tol {tol:g})")
    assert ey <= tol and el <= tol, (tag, ey, el)


# --------------------------------------------------------------- small shapes
@pytest.mark.parametrize("N", [32, 64])
def test_ssd_fp32_ragged(N):
    # 3 chunks (the last 22 steps), 32-channel tiles, h0 given, every option on
    inp = gen.make_ssd_inputs(2, 150, 3, 32, N, io=gen.F32, h0_kind="normal", seed=700 + N)
    check(inp, tag=f"f32-N{N}")


def test_ssd_fp32_16_channel_tiles_options_off():
    # headdim 48 (three 16-channel tiles), one full chunk, no z / D / bias / softplus / h0
    inp = gen.make_ssd_inputs(3, 64, 2, 48, 32, io=gen.F32, h0_kind="none", seed=710, with_z=False,
                              with_D=False, with_bias=False)
    inp["dt"] = (np.abs(inp["dt"]) * np.float32(0.2)).astype(np.float32)
    check(inp, softplus=False, tag="f32-plain")


def test_ssd_fp32_fast_decay():
    # heads with |A| up to e^4: chunk-relative decays underflow inside a chunk
    inp = gen.make_ssd_inputs(1, 200, 4, 32, 64, io=gen.F32, h0_kind="normal", seed=711)
    inp["A"] = (-np.exp(np.array([-4.0, 0.0, 2.5, 4.0]))).astype(np.float32)
    inp["dt_bias"] = np.full(4, 0.5, np.float32)
    check(inp, tag="f32-fast-decay")


@pytest.mark.parametrize("N,P,T", [(64, 64, 300), (128, 32, 130), (32, 16, 65)])
def test_ssd_bf16(N, P, T):
    inp = gen.make_ssd_inputs(2, T, 4, P, N, io=gen.BF16, h0_kind="normal", seed=720 + N + P)
    check(inp, tag=f"bf16-N{N}-P{P}")


# the whole-line kernel (bf16, head sizes that are multiples of 64): every
# d_state, one and two 64-channel tiles per head, ragged and short sequences
@pytest.mark.parametrize("N,P,T", [(64, 64, 300), (64, 128, 129), (32, 64, 65), (128, 128, 200), (32, 192, 1),
                                   (64, 320, 64), (128, 64, 3)])
def test_ssd_bf16_whole_line_tiles(N, P, T):
    inp = gen.make_ssd_inputs(2, T, 3, P, N, io=gen.BF16, h0_kind="normal", seed=750 + N + P + T)
    check(inp, tag=f"bf16-line-N{N}-P{P}-T{T}")


def test_ssd_bf16_whole_line_options_off():
    # no z, D, bias, softplus or h0
    inp = gen.make_ssd_inputs(2, 190, 2, 64, 64, io=gen.BF16, h0_kind="none", seed=760, with_z=False,
                              with_D=False, with_bias=False)
    inp["dt"] = gen.bf16_from_f32(np.abs(gen.f32_from_bf16(inp["dt"])) * np.float32(0.2))
    check(inp, softplus=False, tag="bf16-line-plain")


def test_ssd_bf16_whole_line_fast_decay():
    # heads with |A| up to e^4: decays underflow inside a chunk
    inp = gen.make_ssd_inputs(1, 200, 4, 64, 64, io=gen.BF16, h0_kind="normal", seed=761)
    inp["A"] = (-np.exp(np.array([-4.0, 0.0, 2.5, 4.0]))).astype(np.float32)
    inp["dt_bias"] = np.full(4, 0.5, np.float32)
    check(inp, tag="bf16-line-fast-decay")


@pytest.mark.parametrize("io", [gen.F32, gen.BF16])
def test_ssd_more_workgroups_than_cus(io):
    # 4 x 72 heads x one 32-channel tile = 288 workgroups, more than the CUs:
    # several share a CU; ragged last chunk
    inp = gen.make_ssd_inputs(4, 70, 72, 32, 64, io=io, h0_kind="normal", seed=733)
    check(inp, tag=f"{io}-288wg")


def test_ssd_one_step_and_empty():
    inp = gen.make_ssd_inputs(2, 1, 2, 32, 64, io=gen.F32, h0_kind="normal", seed=730)
    check(inp, tag="T1")
    inp = gen.make_ssd_inputs(2, 0, 2, 32, 64, io=gen.F32, h0_kind="normal", seed=731)
    y, last = run_gpu(inp)
    assert y.size == 0 and np.array_equal(last, inp["h0"].astype(np.float64))


def test_ssd_deterministic_and_continuation():
    from selective_scan_ssm_amd import ops
    inp = gen.make_ssd_inputs(2, 256, 2, 64, 64, io=gen.F32, h0_kind="normal", seed=732)
    y1, l1 = run_gpu(inp)
    y2, l2 = run_gpu(inp)
    assert np.array_equal(y1, y2) and np.array_equal(l1, l2)
    # the same sequence in two calls (split off the 64-step grid), the second from the first's state
    t = {k: G.to_torch(inp[k], gen.F32) for k in IO + F32}
    cut = 100
    a = {k: t[k][:, :cut].contiguous() for k in IO}
    b = {k: t[k][:, cut:].contiguous() for k in IO}
    ya, la = ops.ssd_scan_fwd(a["x"], a["dt"], t["A"], a["B"], a["C"], D=t["D"], z=a["z"], dt_bias=t["dt_bias"],
                              h0=t["h0"], return_last_state=True)
    yb, lb = ops.ssd_scan_fwd(b["x"], b["dt"], t["A"], b["B"], b["C"], D=t["D"], z=b["z"], dt_bias=t["dt_bias"],
                              h0=la, return_last_state=True)
    torch.cuda.synchronize()
    yo, lo = run_oracle(inp)
    ey = G.err(np.concatenate([G.from_torch(ya), G.from_torch(yb)], axis=1), yo)
    el = G.err(G.from_torch(lb), lo)
    G.say(f"[ssd] continuation err_y={ey:.2e} err_last={el:.2e}")
    assert ey <= 1e-5 and el <= 1e-5


def ssd_segments(inp):
    """(segments, chunks per segment) of ssd_scan_fwd's time split for inp's shape."""
    import ctypes
    from selective_scan_ssm_amd import _lib
    S, cps = ctypes.c_int(0), ctypes.c_int(0)
    io = _lib.SSM_BF16 if inp["io"] == gen.BF16 else _lib.SSM_F32
    assert _lib.load().ssm_testing_ssd_segments(inp["batch"], inp["seqlen"], inp["nheads"], inp["headdim"],
                                                inp["d_state"], io, ctypes.byref(S), ctypes.byref(cps)) == 0
    return S.value, cps.value


@pytest.mark.parametrize("N,T,gate", [(32, 4000, True), (64, 2500, False)])
def test_ssd_bf16_time_segments(N, T, gate):
    """The whole-line kernel cut into time segments of several chunks: the
    state pass's segment states and decays carry h0 into every later segment;
    the last segment and the last chunk are ragged."""
    inp = gen.make_ssd_inputs(2, T, 4, 128, N, io=gen.BF16, h0_kind="normal", seed=780 + N, with_z=gate)
    S, cps = ssd_segments(inp)
    assert S > 1 and cps > 1 and (T + 63) // 64 < S * cps, (S, cps)
    check(inp, tag=f"bf16-segments-{S}x{cps}")


def test_ssd_bf16_time_segments_fast_decay_deterministic():
    # |A| up to e^4 (segment decays underflow to 0) and two calls bit for bit
    inp = gen.make_ssd_inputs(1, 3000, 4, 64, 64, io=gen.BF16, h0_kind="normal", seed=790)
    inp["A"] = (-np.exp(np.array([-4.0, 0.0, 2.5, 4.0]))).astype(np.float32)
    inp["dt_bias"] = np.full(4, 0.5, np.float32)
    assert ssd_segments(inp)[0] > 1
    check(inp, tag="bf16-segments-fast-decay")
    y1, l1 = run_gpu(inp)
    y2, l2 = run_gpu(inp)
    assert np.array_equal(y1, y2) and np.array_equal(l1, l2)


# -------------------------------------------------- the layer shapes, full size
@pytest.mark.parametrize("name", ["mamba2-130m-ssd-layer-bf16", "mamba2-2.7b-ssd-layer-bf16"])
def test_ssd_layer_every_output(name):
    """One launch at the full layer shape; every output and final state
    against the oracle."""
    inp = gen.ssd_workload_inputs(name, seed=741)
    if name == "mamba2-2.7b-ssd-layer-bf16":
        assert ssd_segments(inp) == (8, 16)           # the launch the bench times
    G.say(f"[ssd] {name} full size, every output, segments {ssd_segments(inp)}")
    y, last = run_gpu(inp)
    yo, lo = run_oracle(inp)
    ey, el = G.err(y, yo), G.err(last, lo)
    G.say(f"[ssd] {name} all err_y={ey:.2e} err_last={el:.2e}")
    assert ey <= 2e-2 and el <= 2e-2


@pytest.mark.parametrize("name", ["mamba2-130m-ssd-layer-bf16", "mamba2-2.7b-ssd-layer-bf16"])
def test_ssd_layer_full_sampled(name):
    """One launch at the full layer shape; sampled heads x channels (every
    batch row, every step) against the oracle run on exactly those chains."""
    inp = gen.ssd_workload_inputs(name, seed=740)
    G.say(f"[ssd] {name} full size")
    y, last = run_gpu(inp)
    H, P = inp["nheads"], inp["headdim"]
    heads = [0, H // 2, H - 1]
    chans = list(range(0, 8)) + list(range(P - 8, P))
    yo, lo = run_oracle(inp, heads=heads, chans=chans)
    ys = y[:, :, heads][:, :, :, chans]
    ls = last[:, heads][:, :, chans]
    ey, el = G.err(ys, yo), G.err(ls, lo)
    G.say(f"[ssd] {name} sampled err_y={ey:.2e} err_last={el:.2e}")
    assert ey <= 2e-2 and el <= 2e-2
    assert np.all(np.isfinite(y)) and np.all(np.isfinite(last))


def test_ssd_largest_batch_row():
    """One batch row just under the 2 GiB span the kernel's 32-bit buffer
    offsets allow ((seqlen + 128) x heads x head size x 2 bytes < 2^31): 400,000
    steps of the 2.7b layer's width (8 heads x 320, d_state 64), 2.05 GB per
    tensor.  Inputs are drawn on the device (N(0,1) x, dt, z, B, C; A = -exp of
    N(0,1) per head; the S4 dt bias; N(0,1) D and h0); sampled heads x
    channels over the whole sequence are checked against the oracle."""
    from selective_scan_ssm_amd import ops
    Bt, T, H, P, N = 1, 400_000, 8, 320, 64
    assert (T + 128) * H * P * 2 < (1 << 31)
    G.say(f"[ssd] largest batch row: T={T} H={H} P={P} N={N} bf16")
    g = torch.Generator(device="cuda").manual_seed(4202)
    rnd = lambda *s: torch.randn(*s, generator=g, device="cuda", dtype=torch.float32)
    x, z = rnd(Bt, T, H, P).to(torch.bfloat16), rnd(Bt, T, H, P).to(torch.bfloat16)
    dt = rnd(Bt, T, H).to(torch.bfloat16)
    B, C = rnd(Bt, T, N).to(torch.bfloat16), rnd(Bt, T, N).to(torch.bfloat16)
    A = -torch.exp(rnd(H))
    dt0 = torch.exp(torch.rand(H, generator=g, device="cuda") * (np.log(1e-1) - np.log(1e-3)) + np.log(1e-3))
    dt_bias = torch.log(torch.expm1(dt0)).float()
    D, h0 = rnd(H), rnd(Bt, H, P, N)
    y, last = ops.ssd_scan_fwd(x, dt, A, B, C, D=D, z=z, dt_bias=dt_bias, h0=h0, return_last_state=True)
    torch.cuda.synchronize()
    heads, chans = [0, 7], [0, 1, 318, 319]
    sub = lambda t: G.from_torch(t[:, :, heads][:, :, :, chans].contiguous())
    f64 = lambda t: t.detach().cpu().double().numpy()
    yo, lo = oracle.ssd_scan(sub(x), G.from_torch(dt[:, :, heads].contiguous()), f64(A[heads]), G.from_torch(B),
                             G.from_torch(C), D=f64(D[heads]), z=sub(z), dt_bias=f64(dt_bias[heads]),
                             h0=f64(h0[:, heads][:, :, chans]), threads=G.ORACLE_THREADS)
    ey = G.err(sub(y), yo)
    el = G.err(G.from_torch(last[:, heads][:, :, chans].contiguous()), lo)
    G.say(f"[ssd] largest batch row err_y={ey:.2e} err_last={el:.2e}")
    assert ey <= 2e-2 and el <= 2e-2
    assert bool(torch.isfinite(last).all())
