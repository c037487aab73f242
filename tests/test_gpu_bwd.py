"""GPU parity of the backward (ssm_scan_bwd through the C ABI) against the fp64
oracle's gradient (oracle_selective_scan_bwd, pinned by finite differences) on
the same seeded inputs.

Tolerances (max relative error with an rms floor, gpu_util.err):
  * bf16 io: 2e-2 for every gradient, as for the forward;
  * fp32 io: 1e-5 for the per-chain gradients (dx, ddelta, dz, dh0), whose
    arithmetic is one reverse sweep of the same depth as the forward's; 5e-5
    for the gradients summed over the batch, the sequence or the channels (dA,
    dD, ddelta_bias over batch x seqlen terms; dB, dC over d_inner terms).
    Those sums are formed in fp32 in a different order from the oracle's fp64
    ones; with K terms of mixed sign the rounding of such a sum grows like
    sqrt(K) u sum|terms| / |sum|, a few 1e-6 at the sizes below.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import gpu_util as G
import oracle
from selective_scan_ssm_amd import inputs as gen

pytestmark = pytest.mark.gpu

PER_CHAIN = ("dx", "ddelta", "dz", "dh0")
SUMMED = ("dA", "dB", "dC", "dD", "ddelta_bias")
TOL_F32_SUMMED = 5e-5


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from selective_scan_ssm_amd import _lib
    _lib.load()
    assert len(_lib.hip_runtimes_mapped()) == 1


def grads_inputs(inp, seed, with_dlast=True):
    """dL/dy in the io dtype (as stored) and dL/dlast_state in fp32."""
    rng = np.random.default_rng(seed)
    dout = rng.standard_normal(inp["x"].shape).astype(np.float32)
    if inp["io"] == gen.BF16:
        dout = gen.bf16_from_f32(dout)
    dlast = rng.standard_normal((inp["batch"], inp["d_inner"], inp["d_state"])).astype(np.float32) \
        if with_dlast else None
    return dout, dlast


def run_bwd_gpu(inp, dout, dlast, softplus=True):
    from selective_scan_ssm_amd import ops
    t = G.device_inputs(inp)
    g = ops.scan_bwd(t["x"], t["delta"], t["A"], t["B"], t["C"], G.to_torch(dout, inp["io"]),
                     D=t["D"], z=t["z"], delta_bias=t["delta_bias"], delta_softplus=softplus,
                     h0=t["h0"], dlast=G.to_torch(dlast, gen.F32))
    torch.cuda.synchronize()
    return {k: G.from_torch(v) for k, v in g.items()}


def run_bwd_oracle(inp, dout, dlast, softplus=True, d_index=None, b_index=None):
    d = G.decoded(inp)
    go = gen.to_f64(dout, inp["io"])
    dl = None if dlast is None else np.asarray(dlast, np.float64)
    if b_index is not None:
        bi = np.asarray(b_index)
        pick = lambda a: None if a is None else np.ascontiguousarray(a[bi])
        d = dict(d, x=pick(d["x"]), delta=pick(d["delta"]), z=pick(d["z"]), B=pick(d["B"]),
                 C=pick(d["C"]), h0=pick(d["h0"]))
        go, dl = pick(go), pick(dl)
    if d_index is not None:
        di = np.asarray(d_index)
        sl = lambda a: None if a is None else np.ascontiguousarray(a[:, :, di])
        d = dict(d, x=sl(d["x"]), delta=sl(d["delta"]), z=sl(d["z"]), A=d["A"][di],
                 D=None if d["D"] is None else d["D"][di],
                 delta_bias=None if d["delta_bias"] is None else d["delta_bias"][di],
                 h0=None if d["h0"] is None else np.ascontiguousarray(d["h0"][:, di]))
        go = np.ascontiguousarray(go[:, :, di])
        dl = None if dl is None else np.ascontiguousarray(dl[:, di])
    return oracle.selective_scan_bwd(d["x"], d["delta"], d["A"], d["B"], d["C"], go, D=d["D"],
                                     z=d["z"], delta_bias=d["delta_bias"], delta_softplus=softplus,
                                     h0=d["h0"], dlast=dl, threads=G.ORACLE_THREADS)


def tol_for(io, key):
    if io == gen.BF16:
        return 2e-2
    return 1e-5 if key in PER_CHAIN else TOL_F32_SUMMED


def compare(g, o, io, keys, tag):
    worst = {}
    for k in keys:
        if o.get(k) is None:
            assert g.get(k) is None, k
            continue
        e = G.err(g[k], o[k])
        worst[k] = e
    G.say(f"[bwd] {tag} " + " ".join(f"{k}={v:.2e}" for k, v in worst.items()))
    for k, e in worst.items():
        assert e <= tol_for(io, k), (tag, k, e)


def segments(inp):
    """(segments, blocks per segment) of the backward's time split for inp's shape."""
    import ctypes
    from selective_scan_ssm_amd import _lib
    S, sblk = ctypes.c_int(0), ctypes.c_int(0)
    io = _lib.SSM_BF16 if inp["io"] == gen.BF16 else _lib.SSM_F32
    assert _lib.load().ssm_testing_bwd_segments(inp["batch"], inp["seqlen"], inp["d_inner"], inp["d_state"],
                                                io, ctypes.byref(S), ctypes.byref(sblk)) == 0
    return S.value, sblk.value


def check_bwd(inp, softplus=True, with_dlast=True, seed=0, tag=""):
    G.say(f"[bwd] {tag} B={inp['batch']} T={inp['seqlen']} D={inp['d_inner']} N={inp['d_state']} "
          f"io={inp['io']} segments={segments(inp)}")
    dout, dlast = grads_inputs(inp, seed, with_dlast)
    g = run_bwd_gpu(inp, dout, dlast, softplus)
    o = run_bwd_oracle(inp, dout, dlast, softplus)
    compare(g, o, inp["io"], PER_CHAIN + SUMMED, tag)


# --------------------------------------------------------------- small shapes
@pytest.mark.parametrize("N", [1, 3, 4, 5, 9, 16])
def test_bwd_fp32_every_width(N):
    # 3 channel tiles (the last ragged), 7 blocks of 16 steps (the last ragged)
    inp = gen.make_inputs(2, 100, 130, N, io=gen.F32, a_kind="sm1", h0_kind="normal", seed=400 + N)
    check_bwd(inp, seed=N, tag=f"f32-N{N}")


def test_bwd_bf16_mamba_layer_shape():
    inp = gen.make_inputs(2, 300, 200, 16, io=gen.BF16, seed=411)
    check_bwd(inp, seed=11, tag="bf16-N16")


def test_bwd_options_off():
    # no gate, no D, no bias, softplus off (positive Delta), no h0, no dL/dlast
    inp = gen.make_inputs(1, 77, 70, 16, io=gen.F32, seed=412, with_z=False, with_D=False,
                          with_bias=False)
    inp["delta"] = (np.abs(inp["delta"]) * np.float32(0.05)).astype(np.float32)
    check_bwd(inp, softplus=False, with_dlast=False, seed=12, tag="f32-plain")


def test_bwd_sm1_shape_long():
    # d_state 1 over a long sequence (the SM1 distributions: fast decays, h0 ~ N(0,1))
    inp = gen.make_inputs(2, 1000, 96, 1, io=gen.F32, a_kind="sm1", h0_kind="normal", seed=413)
    check_bwd(inp, seed=13, tag="f32-sm1-long")


@pytest.mark.parametrize("T,io", [(16, gen.F32), (9, gen.BF16)])
def test_bwd_one_segment(T, io):
    # a sequence of one block is swept by one segment (no carry pass)
    inp = gen.make_inputs(2, T, 130, 16, io=io, h0_kind="normal", seed=416 + T)
    assert segments(inp)[0] == 1
    check_bwd(inp, seed=16 + T, tag=f"one-segment-T{T}")


@pytest.mark.parametrize("T,io,N", [(1000, gen.F32, 16), (4000, gen.BF16, 16), (1500, gen.F32, 5)])
def test_bwd_many_segments(T, io, N):
    # long rows of few tiles: many segments, the last one ragged, so every
    # segment's incoming adjoint comes through the carry pass; A = -(n+1)
    # and the SM1 draw A = -exp(U(-4, 1)) (decays as slow as 0.018 per unit Delta)
    inp = gen.make_inputs(1, T, 70, N, io=io, a_kind="sm1" if N != 16 else "hippo", h0_kind="normal",
                          seed=430 + N)
    S, sblk = segments(inp)
    assert S > 8 and S * sblk * 16 > T, (S, sblk)
    check_bwd(inp, seed=30 + N, tag=f"segments-{S}x{sblk}")


def test_bwd_empty_sequence():
    inp = gen.make_inputs(2, 0, 70, 16, io=gen.F32, h0_kind="normal", seed=414)
    dout, dlast = grads_inputs(inp, 14)
    g = run_bwd_gpu(inp, dout, dlast)
    assert np.array_equal(g["dh0"], dlast.astype(np.float64))
    assert not g["dA"].any() and not g["dD"].any() and not g["ddelta_bias"].any()


def test_bwd_deterministic():
    inp = gen.make_inputs(2, 64, 130, 16, io=gen.BF16, seed=415)
    dout, dlast = grads_inputs(inp, 15)
    g1 = run_bwd_gpu(inp, dout, dlast)
    g2 = run_bwd_gpu(inp, dout, dlast)
    for k, v in g1.items():
        if v is not None:
            assert np.array_equal(v, g2[k]), k


# -------------------------------------------------- the layer shapes, full size
def test_bwd_mamba130m_layer_full_row0():
    """The 130m-shaped layer (batch 8, seqlen 2048, d_inner 1536, d_state 16,
    bf16) in one launch; batch row 0 checked in full (every channel, so dB, dC
    of that row too) against the oracle run on that row."""
    inp = gen.workload_inputs(2)
    dout, dlast = grads_inputs(inp, 21)
    g = run_bwd_gpu(inp, dout, dlast)
    o = run_bwd_oracle(inp, dout, dlast, b_index=[0])
    row0 = {k: (None if g[k] is None else g[k][:1]) for k in ("dx", "ddelta", "dz", "dh0", "dB", "dC")}
    compare(row0, o, gen.BF16, ("dx", "ddelta", "dz", "dh0", "dB", "dC"), "w2-row0")
    for k in ("dA", "dD", "ddelta_bias"):
        assert np.all(np.isfinite(g[k])), k


def test_bwd_mamba2p8b_layer_full_sampled():
    """The 2.8b-shaped layer (batch 4, seqlen 8192, d_inner 5120, d_state 16,
    bf16) in one launch; the per-chain gradients and dA, dD, ddelta_bias of
    sampled channels against the oracle run on those channels."""
    inp = gen.workload_inputs(3)
    dout, dlast = grads_inputs(inp, 22)
    g = run_bwd_gpu(inp, dout, dlast)
    d_index = np.r_[0:8, 2560:2568, 5112:5120]
    o = run_bwd_oracle(inp, dout, dlast, d_index=d_index)
    sub = dict(dx=g["dx"][:, :, d_index], ddelta=g["ddelta"][:, :, d_index], dz=g["dz"][:, :, d_index],
               dh0=g["dh0"][:, d_index], dA=g["dA"][d_index], dD=g["dD"][d_index],
               ddelta_bias=g["ddelta_bias"][d_index])
    compare(sub, o, gen.BF16, ("dx", "ddelta", "dz", "dh0", "dA", "dD", "ddelta_bias"), "w3-sampled")
    for k in ("dB", "dC"):
        assert np.all(np.isfinite(g[k])), k


def test_bwd_largest_batch_row():
    """One batch row just under the 2 GiB span the backward's 32-bit offsets
    allow (seqlen x d_inner x 2 bytes < 2^31): 200,000 steps x 5120 channels,
    d_state 16, bf16, 2.05 GB per tensor.  Inputs drawn on the device (N(0,1)
    x, delta, z, B, C, dL/dy; A = -(n+1); S4 delta bias; N(0,1) D, h0 and
    dL/dlast); the per-chain gradients and dA, dD, ddelta_bias of sampled
    channels against the oracle run on those channels (dB and dC sum over
    every channel: checked finite)."""
    from selective_scan_ssm_amd import ops
    Bt, T, Dd, N = 1, 200_000, 5120, 16
    assert T * Dd * 2 < (1 << 31)
    G.say(f"[bwd] largest batch row: T={T} D={Dd} N={N} bf16")
    g = torch.Generator(device="cuda").manual_seed(4203)
    rnd = lambda *s: torch.randn(*s, generator=g, device="cuda", dtype=torch.float32)
    x, dl, z, dy = (rnd(Bt, T, Dd).to(torch.bfloat16) for _ in range(4))
    B, C = rnd(Bt, T, N).to(torch.bfloat16), rnd(Bt, T, N).to(torch.bfloat16)
    A = -(torch.arange(N, device="cuda", dtype=torch.float32) + 1.0).expand(Dd, N).contiguous()
    dt0 = torch.exp(torch.rand(Dd, generator=g, device="cuda") * (np.log(1e-1) - np.log(1e-3)) + np.log(1e-3))
    bias = torch.log(torch.expm1(dt0)).float()
    D, h0, dlast = rnd(Dd), rnd(Bt, Dd, N), rnd(Bt, Dd, N)
    gr = ops.scan_bwd(x, dl, A, B, C, dy, D=D, z=z, delta_bias=bias, h0=h0, dlast=dlast)
    torch.cuda.synchronize()
    di = np.r_[0:4, 2558:2562, 5116:5120]
    col = lambda t: G.from_torch(t[:, :, di].contiguous())
    f64 = lambda t: t.detach().cpu().double().numpy()
    o = oracle.selective_scan_bwd(col(x), col(dl), f64(A[di]), G.from_torch(B), G.from_torch(C), col(dy),
                                  D=f64(D[di]), z=col(z), delta_bias=f64(bias[di]), h0=f64(h0[:, di]),
                                  dlast=f64(dlast[:, di]), threads=G.ORACLE_THREADS)
    sub = dict(dx=col(gr["dx"]), ddelta=col(gr["ddelta"]), dz=col(gr["dz"]),
               dh0=G.from_torch(gr["dh0"][:, di].contiguous()), dA=G.from_torch(gr["dA"][di].contiguous()),
               dD=G.from_torch(gr["dD"][di].contiguous()), ddelta_bias=G.from_torch(gr["ddelta_bias"][di].contiguous()))
    compare(sub, o, gen.BF16, ("dx", "ddelta", "dz", "dh0", "dA", "dD", "ddelta_bias"), "largest-row")
    for k in ("dB", "dC"):
        assert bool(torch.isfinite(gr[k]).all()), k


@pytest.mark.parametrize("io,N,T", [(gen.BF16, 16, 300), (gen.F32, 16, 75), (gen.F32, 4, 130), (gen.BF16, 7, 40)])
def test_bwd_with_forward_checkpoints(io, N, T):
    """ssm_scan_fwd_ckpt + ssm_scan_bwd_ckpt: the forward's y and last_state
    are those of ssm_scan_fwd and the gradients those of ssm_scan_bwd, bit for
    bit; the checkpoint of block j is the state after the first 16 j steps
    (the oracle's last_state of that prefix)."""
    from selective_scan_ssm_amd import ops
    inp = gen.make_inputs(2, T, 200, N, io=io, a_kind="sm1", h0_kind="normal", seed=340 + N)
    t = G.device_inputs(inp)
    kw = dict(D=t["D"], z=t["z"], delta_bias=t["delta_bias"], h0=t["h0"])
    y1, l1 = ops.scan_fwd(t["x"], t["delta"], t["A"], t["B"], t["C"], return_last_state=True, **kw)
    ck = torch.empty(ops.ckpt_shape(2, T, 200, N), dtype=torch.float32, device="cuda")
    y2, l2 = ops.scan_fwd(t["x"], t["delta"], t["A"], t["B"], t["C"], return_last_state=True, ckpt_out=ck, **kw)
    dout, dlast = grads_inputs(inp, 41)
    dd, dl = G.to_torch(dout, io), G.to_torch(dlast, gen.F32)
    g1 = ops.scan_bwd(t["x"], t["delta"], t["A"], t["B"], t["C"], dd, dlast=dl, **kw)
    g2 = ops.scan_bwd(t["x"], t["delta"], t["A"], t["B"], t["C"], dd, dlast=dl, ckpt=ck, **kw)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(l1, l2)
    for k in g1:
        if g1[k] is not None:
            assert torch.equal(g1[k], g2[k]), k
    c = G.from_torch(ck)
    assert np.array_equal(c[:, 0], inp["h0"].astype(np.float64))
    d = G.decoded(inp)
    for j in (1, (T - 1) // 16):
        s = 16 * j
        pre = lambda a: None if a is None else np.ascontiguousarray(a[:, :s])
        _, lo = oracle.selective_scan(pre(d["x"]), pre(d["delta"]), d["A"], pre(d["B"]), pre(d["C"]), D=d["D"],
                                      z=pre(d["z"]), delta_bias=d["delta_bias"], h0=d["h0"],
                                      threads=G.ORACLE_THREADS)
        e = G.err(c[:, j], lo)
        G.say(f"[bwd] checkpoint block {j} ({io}, N={N}) err={e:.2e}")
        assert e <= (1e-5 if io == gen.F32 else 2e-2), (j, e)


def test_bwd_concurrent_host_threads():
    """Self-contained backward calls from four host threads, each on a stream
    of its own, at once: they share the library's side stream per device (the
    carry pass beside the checkpoint pass), whose fork and join are enqueued
    under a lock.  Every call's gradients equal those of a call made alone,
    bit for bit."""
    import threading
    from selective_scan_ssm_amd import ops
    inputs = [gen.make_inputs(2, 700, 260, 16, io=gen.BF16, h0_kind="normal", seed=480 + i) for i in range(4)]
    assert all(segments(inp)[0] > 1 for inp in inputs)
    dev = [G.device_inputs(inp) for inp in inputs]
    douts = [G.to_torch(grads_inputs(inp, 80 + i)[0], inp["io"]) for i, inp in enumerate(inputs)]
    call = lambda t, d: ops.scan_bwd(t["x"], t["delta"], t["A"], t["B"], t["C"], d, D=t["D"], z=t["z"],
                                     delta_bias=t["delta_bias"], h0=t["h0"])
    alone = []
    for t, d in zip(dev, douts):
        alone.append(call(t, d))
        torch.cuda.synchronize()
    results, errors = [None] * 4, []

    def worker(i):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                for _ in range(3):
                    results[i] = call(dev[i], douts[i])
            s.synchronize()
        except Exception as e:          # reported below
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(4)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for i in range(4):
        for k, v in alone[i].items():
            if v is not None:
                assert torch.equal(v, results[i][k]), (i, k)
