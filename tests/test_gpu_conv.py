"""GPU parity of the causal depthwise conv1d (+ SiLU) and its decode update
(through the C ABI) against the fp64 oracle on the same seeded inputs.
Tolerance as for the scan outputs: 1e-5 fp32, 2e-2 bf16 (gpu_util.err)."""
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


def case(io, Bt, T, Dd, K, seed, with_state=True, with_bias=True):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((Bt, T, Dd)).astype(np.float32)
    st = rng.standard_normal((Bt, Dd, K - 1)).astype(np.float32) if with_state else None
    if io == gen.BF16:
        x = gen.bf16_from_f32(x)
        st = None if st is None else gen.bf16_from_f32(st)
    w = (rng.standard_normal((Dd, K)) * 0.5).astype(np.float32)
    bias = rng.standard_normal(Dd).astype(np.float32) if with_bias else None
    return x, w, bias, st


def run_case(io, Bt, T, Dd, K, seed, silu=True, with_state=True, with_bias=True, tag=""):
    from selective_scan_ssm_amd import ops
    x, w, bias, st = case(io, Bt, T, Dd, K, seed, with_state, with_bias)
    G.say(f"[conv] {tag} B={Bt} T={T} D={Dd} K={K} io={io} state={with_state} silu={silu}")
    out, so = ops.causal_conv1d(G.to_torch(x, io), G.to_torch(w, gen.F32), G.to_torch(bias, gen.F32),
                                conv_state=G.to_torch(st, io), silu=silu, return_state=True)
    torch.cuda.synchronize()
    oo, oso = oracle.causal_conv1d(gen.to_f64(x, io), w, bias, None if st is None else gen.to_f64(st, io),
                                   silu=silu, threads=G.ORACLE_THREADS)
    e = G.err(G.from_torch(out), oo)
    tol = G.TOL[io]
    G.say(f"[conv] {tag} err={e:.2e} tol={tol:g}")
    assert e <= tol
    # the state after the sequence is a copy of inputs: bit-exact
    assert np.array_equal(G.from_torch(so), oso)


@pytest.mark.parametrize("io", [gen.F32, gen.BF16])
@pytest.mark.parametrize("K", [1, 2, 3, 4])
def test_conv_widths(io, K):
    # d_inner % 4 == 0: the 4-channel vector path; ragged chunks and sequence
    run_case(io, 2, 300, 520, K, 500 + K, tag=f"K{K}")


@pytest.mark.parametrize("io", [gen.F32, gen.BF16])
def test_conv_scalar_path(io):
    # d_inner not a multiple of 4: one channel per lane
    run_case(io, 3, 129, 101, 4, 510, tag="scalar")


def test_conv_short_and_plain():
    run_case(gen.F32, 2, 2, 64, 4, 511, with_state=True, tag="T<K")        # window keeps old inputs
    run_case(gen.F32, 1, 50, 64, 4, 512, silu=False, with_state=False, with_bias=False, tag="plain")
    run_case(gen.BF16, 1, 0, 64, 4, 513, tag="T=0")


def test_conv_update_matches_oracle_and_sequence():
    from selective_scan_ssm_amd import ops
    for io in (gen.F32, gen.BF16):
        x, w, bias, st = case(io, 4, 6, 200, 4, 520)
        stt = G.to_torch(st, io).clone()
        wt, bt = G.to_torch(w, gen.F32), G.to_torch(bias, gen.F32)
        ost = gen.to_f64(st, io)
        outs = []
        for t in range(6):
            xt = G.to_torch(np.ascontiguousarray(x[:, t]), io)
            outs.append(G.from_torch(ops.causal_conv1d_update(stt, xt, wt, bt, silu=True)))
            oo, ost = oracle.conv1d_update(ost, gen.to_f64(np.ascontiguousarray(x[:, t]), io), w, bias, silu=True)
            assert G.err(outs[-1], oo) <= G.TOL[io]
        torch.cuda.synchronize()
        assert np.array_equal(G.from_torch(stt), ost)
        # six decode tokens = the whole-sequence convolution from the same state
        full, _ = oracle.causal_conv1d(gen.to_f64(x, io), w, bias, gen.to_f64(st, io), silu=True)
        assert G.err(np.stack(outs, axis=1), full) <= G.TOL[io]


def test_conv_mamba2p8b_shape_sampled():
    """The 2.8b layer's x (batch 4, seqlen 8192, d_inner 5120, bf16, width 4) in
    one launch; sampled channels against the oracle."""
    from selective_scan_ssm_amd import ops
    x, w, bias, st = case(gen.BF16, 4, 8192, 5120, 4, 530, with_state=False)
    out = ops.causal_conv1d(G.to_torch(x, gen.BF16), G.to_torch(w, gen.F32), G.to_torch(bias, gen.F32))
    torch.cuda.synchronize()
    di = np.r_[0:8, 2600:2608, 5112:5120]
    oo, _ = oracle.causal_conv1d(gen.to_f64(np.ascontiguousarray(x[:, :, di]), gen.BF16), w[di], bias[di],
                                 None, silu=True, threads=G.ORACLE_THREADS)
    e = G.err(G.from_torch(out)[:, :, di], oo)
    G.say(f"[conv] w3-shape sampled err={e:.2e}")
    assert e <= 2e-2


def test_conv_largest_batch_row():
    """One batch row just under the 2 GiB span of 32-bit offsets (seqlen x
    d_inner x 2 bytes < 2^31): 200,000 steps x 5120 channels, bf16, width 4,
    with an incoming window; drawn on the device; sampled channels over the
    whole sequence against the oracle, the outgoing window exactly."""
    from selective_scan_ssm_amd import ops
    Bt, T, Dd, K = 1, 200_000, 5120, 4
    assert T * Dd * 2 < (1 << 31)
    G.say(f"[conv] largest batch row: T={T} D={Dd} width={K} bf16")
    g = torch.Generator(device="cuda").manual_seed(4204)
    x = torch.randn(Bt, T, Dd, generator=g, device="cuda").to(torch.bfloat16)
    st = torch.randn(Bt, Dd, K - 1, generator=g, device="cuda").to(torch.bfloat16)
    w = torch.randn(Dd, K, generator=g, device="cuda") * 0.5
    b = torch.randn(Dd, generator=g, device="cuda")
    out, so = ops.causal_conv1d(x, w, b, conv_state=st, silu=True, return_state=True)
    torch.cuda.synchronize()
    di = np.r_[0:4, 2558:2562, 5116:5120]
    oo, oso = oracle.causal_conv1d(G.from_torch(x[:, :, di].contiguous()), w[di].cpu().double().numpy(),
                                   b[di].cpu().double().numpy(), G.from_torch(st[:, di].contiguous()), silu=True,
                                   threads=G.ORACLE_THREADS)
    e = G.err(G.from_torch(out[:, :, di].contiguous()), oo)
    G.say(f"[conv] largest batch row err={e:.2e}")
    assert e <= 2e-2
    assert np.array_equal(G.from_torch(so[:, di].contiguous()), oso)
