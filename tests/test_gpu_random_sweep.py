"""Seeded random sweeps of every entry point against the fp64 oracle: small
shapes whose sizes, dtypes and optional inputs are drawn together, so that
combinations no hand-picked case names (a ragged tail with softplus off and no
gate, a one-step sequence with an initial state, ...) are exercised too.  The
draws are fixed by the case number; each case prints its parameters before it
runs.  Tolerances as everywhere (gpu_util.err): 1e-5 fp32, 2e-2 bf16 (the
backward's summed gradients 5e-5 in fp32, as in test_gpu_bwd)."""
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


def draw(case, salt):
    return np.random.default_rng(np.random.SeedSequence([9000 + salt, case]))


# ------------------------------------------------------------- forward scan
@pytest.mark.parametrize("case", range(12))
def test_scan_random(case):
    r = draw(case, 1)
    io = gen.BF16 if r.random() < 0.5 else gen.F32
    Bt, T, Dd, N = int(r.integers(1, 4)), int(r.integers(1, 300)), int(r.integers(1, 200)), int(r.integers(1, 17))
    opts = dict(with_z=bool(r.random() < 0.7), with_D=bool(r.random() < 0.7), with_bias=bool(r.random() < 0.7))
    h0_kind = ["none", "zero", "normal"][int(r.integers(0, 3))]
    softplus = bool(r.random() < 0.75)
    if not softplus:  # without softplus the step is the raw input: keep it >= 0 (no negative bias)
        opts["with_bias"] = False
    G.say(f"[sweep] scan case {case}: B={Bt} T={T} D={Dd} N={N} io={io} {opts} h0={h0_kind} softplus={softplus}")
    inp = gen.make_inputs(Bt, T, Dd, N, io=io, a_kind="sm1" if r.random() < 0.5 else "hippo", h0_kind=h0_kind,
                          seed=100 + case, **opts)
    if not softplus:
        inp["delta"] = gen.bf16_from_f32(np.abs(gen.f32_from_bf16(inp["delta"])) * np.float32(0.3)) \
            if io == gen.BF16 else (np.abs(inp["delta"]) * np.float32(0.3)).astype(np.float32)
    y, last = G.run_scan(inp, softplus=softplus)
    yo, lo = G.run_oracle(inp, softplus=softplus)
    ey, el = G.err(y, yo), G.err(last, lo)
    G.say(f"[sweep] scan case {case}: err_y={ey:.2e} err_last={el:.2e}")
    assert ey <= G.TOL[io] and el <= G.TOL[io]


# ------------------------------------------------------------ Mamba-2 (SSD)
@pytest.mark.parametrize("case", range(10))
def test_ssd_random(case):
    from selective_scan_ssm_amd import ops
    r = draw(case, 2)
    io = gen.BF16 if r.random() < 0.5 else gen.F32
    Bt, T, H = int(r.integers(1, 4)), int(r.integers(1, 200)), int(r.integers(1, 6))
    P = int(r.choice([16, 32, 48, 64, 96]))
    N = int(r.choice([32, 64, 128] if io == gen.BF16 else [32, 64]))
    opts = dict(with_z=bool(r.random() < 0.7), with_D=bool(r.random() < 0.7), with_bias=bool(r.random() < 0.7))
    h0_kind = ["none", "zero", "normal"][int(r.integers(0, 3))]
    softplus = bool(r.random() < 0.75)
    if not softplus:
        opts["with_bias"] = False
    G.say(f"[sweep] ssd case {case}: B={Bt} T={T} H={H} P={P} N={N} io={io} {opts} h0={h0_kind} softplus={softplus}")
    inp = gen.make_ssd_inputs(Bt, T, H, P, N, io=io, h0_kind=h0_kind, seed=200 + case, **opts)
    if not softplus:
        a = np.abs(gen.to_f64(inp["dt"], io)).astype(np.float32) * np.float32(0.3)
        inp["dt"] = gen.bf16_from_f32(a) if io == gen.BF16 else a
    t = {k: G.to_torch(inp[k], io) for k in ("x", "dt", "z", "B", "C")}
    t.update({k: G.to_torch(inp[k], gen.F32) for k in ("A", "D", "dt_bias", "h0")})
    y, last = ops.ssd_scan_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"], dt_bias=t["dt_bias"],
                               dt_softplus=softplus, h0=t["h0"], return_last_state=True)
    torch.cuda.synchronize()
    d = {k: (None if inp[k] is None else gen.to_f64(inp[k], io)) for k in ("x", "dt", "z", "B", "C")}
    yo, lo = oracle.ssd_scan(d["x"], d["dt"], inp["A"], d["B"], d["C"], D=inp["D"], z=d["z"],
                             dt_bias=inp["dt_bias"], dt_softplus=softplus, h0=inp["h0"], threads=G.ORACLE_THREADS)
    ey, el = G.err(G.from_torch(y), yo), G.err(G.from_torch(last), lo)
    G.say(f"[sweep] ssd case {case}: err_y={ey:.2e} err_last={el:.2e}")
    assert ey <= G.TOL[io] and el <= G.TOL[io]


# ---------------------------------------------------------------- backward
@pytest.mark.parametrize("case", range(6))
def test_bwd_random(case):
    import test_gpu_bwd as TB
    r = draw(case, 3)
    io = gen.BF16 if r.random() < 0.5 else gen.F32
    Bt, T, Dd, N = int(r.integers(1, 3)), int(r.integers(1, 150)), int(r.integers(1, 140)), int(r.integers(1, 17))
    opts = dict(with_z=bool(r.random() < 0.7), with_D=bool(r.random() < 0.7), with_bias=bool(r.random() < 0.7))
    h0_kind = ["none", "normal"][int(r.integers(0, 2))]
    inp = gen.make_inputs(Bt, T, Dd, N, io=io, a_kind="sm1", h0_kind=h0_kind, seed=300 + case, **opts)
    TB.check_bwd(inp, with_dlast=bool(r.random() < 0.5), seed=case, tag=f"sweep case {case} {opts}")


# --------------------------------------------------------- conv1d + decode
@pytest.mark.parametrize("case", range(8))
def test_conv_random(case):
    from selective_scan_ssm_amd import ops
    r = draw(case, 4)
    io = gen.BF16 if r.random() < 0.5 else gen.F32
    Bt, T, Dd, K = int(r.integers(1, 4)), int(r.integers(1, 300)), int(r.integers(1, 300)), int(r.integers(1, 5))
    silu = bool(r.random() < 0.7)
    with_bias, with_state = bool(r.random() < 0.7), bool(r.random() < 0.5)
    G.say(f"[sweep] conv case {case}: B={Bt} T={T} D={Dd} K={K} io={io} silu={silu} bias={with_bias} "
          f"state={with_state}")
    x = r.standard_normal((Bt, T, Dd)).astype(np.float32)
    wt = (r.standard_normal((Dd, K)) * 0.5).astype(np.float32)
    bias = r.standard_normal(Dd).astype(np.float32) if with_bias else None
    st = r.standard_normal((Bt, Dd, K - 1)).astype(np.float32) if (with_state and K > 1) else None
    if io == gen.BF16:
        x = gen.bf16_from_f32(x)
        st = None if st is None else gen.bf16_from_f32(st)
    out, sto = ops.causal_conv1d(G.to_torch(x, io), G.to_torch(wt, gen.F32), G.to_torch(bias, gen.F32), silu=silu,
                                 conv_state=G.to_torch(st, io), return_state=True)
    torch.cuda.synchronize()
    oo, so = oracle.causal_conv1d(gen.to_f64(x, io), wt, bias, None if st is None else gen.to_f64(st, io),
                                  silu=silu)
    eo = G.err(G.from_torch(out), oo)
    es = 0.0 if K == 1 else G.err(G.from_torch(sto), so)
    G.say(f"[sweep] conv case {case}: err_out={eo:.2e} err_state={es:.2e}")
    assert eo <= G.TOL[io] and es == 0.0


# ------------------------------------------------------------ 2-D orders
@pytest.mark.parametrize("case", range(6))
def test_scan2d_random(case):
    from selective_scan_ssm_amd import ops
    r = draw(case, 5)
    io = gen.BF16 if r.random() < 0.5 else gen.F32
    Hh, Ww = int(r.integers(1, 12)), int(r.integers(1, 12))
    Bt, Dd, N, direction = int(r.integers(1, 3)), int(r.integers(1, 100)), int(r.integers(1, 17)), int(r.integers(0, 4))
    G.say(f"[sweep] 2d case {case}: B={Bt} grid={Hh}x{Ww} D={Dd} N={N} dir={direction} io={io}")
    inp = gen.make_inputs(Bt, Hh * Ww, Dd, N, io=io, a_kind="sm1", h0_kind="normal", seed=500 + case)
    t = G.device_inputs(inp)
    y, last = ops.scan_fwd_2d(t["x"], t["delta"], t["A"], t["B"], t["C"], Hh, Ww, direction, D=t["D"], z=t["z"],
                              delta_bias=t["delta_bias"], h0=t["h0"], return_last_state=True)
    torch.cuda.synchronize()
    d = G.decoded(inp)
    yo, lo = oracle.scan_2d(d["x"], d["delta"], d["A"], d["B"], d["C"], Hh, Ww, direction, D=d["D"], z=d["z"],
                            delta_bias=d["delta_bias"], h0=d["h0"], threads=G.ORACLE_THREADS)
    ey, el = G.err(G.from_torch(y), yo), G.err(G.from_torch(last), lo)
    G.say(f"[sweep] 2d case {case}: err_y={ey:.2e} err_last={el:.2e}")
    assert ey <= G.TOL[io] and el <= G.TOL[io]


# ------------------------------------------------------------ dt_proj
@pytest.mark.parametrize("case", range(8))
def test_dtproj_random(case):
    from selective_scan_ssm_amd import ops
    r = draw(case, 6)
    io = gen.BF16 if r.random() < 0.5 else gen.F32
    pe = 8 if io == gen.BF16 else 4
    rows, rank, dim = int(r.integers(1, 700)), pe * int(r.integers(1, 30)), 4 * int(r.integers(1, 200))
    ldx = rank + pe * int(r.integers(0, 12))
    G.say(f"[sweep] dt_proj case {case}: rows={rows} rank={rank} dim={dim} ldx={ldx} io={io}")
    inp = gen.make_dtproj_inputs(rows, rank, dim, ldx, io=io, seed=600 + case)
    got = ops.dt_proj(G.to_torch(inp["x_dbl"], io)[:, :rank], G.to_torch(inp["W"], io))
    torch.cuda.synchronize()
    e = G.err(G.from_torch(got), oracle.dt_proj(gen.to_f64(inp["x_dbl"], io), gen.to_f64(inp["W"], io)))
    G.say(f"[sweep] dt_proj case {case}: err={e:.2e}")
    assert e <= G.TOL[io]
