"""The fp64 oracle against facts that do not come from itself (see oracle_pins)."""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
import oracle_pins as P
from selective_scan_ssm_amd import inputs as gen


@pytest.fixture(scope="module")
def lib():
    return oracle.load()


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(lib, pin):
    pin(lib)


@settings(max_examples=40, deadline=None)
@given(Bt=st.integers(1, 2), T=st.integers(0, 10), Dd=st.integers(1, 4), N=st.integers(1, 5),
       seed=st.integers(0, 10_000), softplus=st.booleans(), use_z=st.booleans(),
       use_D=st.booleans(), use_bias=st.booleans(), h0_kind=st.sampled_from(["none", "normal"]))
def test_bruteforce_fuzz(lib, Bt, T, Dd, N, seed, softplus, use_z, use_D, use_bias, h0_kind):
    i = gen.make_inputs(Bt, T, Dd, N, io=gen.F32, a_kind="sm1", h0_kind=h0_kind, seed=seed,
                        with_z=use_z, with_D=use_D, with_bias=use_bias)
    if not softplus:
        i["delta"] = np.abs(i["delta"]) * 0.5
    y, last = oracle.selective_scan(i["x"], i["delta"], i["A"], i["B"], i["C"], D=i["D"], z=i["z"],
                                    delta_bias=i["delta_bias"], delta_softplus=softplus,
                                    h0=i["h0"], lib=lib)
    yb, lb = P.brute_force(i["x"], i["delta"], i["A"], i["B"], i["C"], i["D"], i["z"],
                           i["delta_bias"], softplus, i["h0"])
    assert P._rel(y, yb) < 1e-12
    assert P._rel(last, lb) < 1e-12


def test_threads_bitwise_equal(lib):
    i = gen.workload_inputs(2, batch=2, seqlen=64, d_inner=96)
    dec = {k: (gen.to_f64(v, gen.BF16) if k in ("x", "delta", "z", "B", "C") else v)
           for k, v in i.items()}
    args = (dec["x"], dec["delta"], dec["A"], dec["B"], dec["C"])
    kw = dict(D=dec["D"], z=dec["z"], delta_bias=dec["delta_bias"], lib=lib)
    y1, l1 = oracle.selective_scan(*args, threads=1, **kw)
    y4, l4 = oracle.selective_scan(*args, threads=4, **kw)
    assert np.array_equal(y1, y4) and np.array_equal(l1, l4)


@pytest.mark.slow
def test_sm1_closed_form_full_length(lib):
    """Full SM1 sequence length (4096) on a few channels."""
    i = gen.workload_inputs(1, d_inner=8)
    y, last = oracle.sm1_scan(i["x"], i["delta"], i["A"][:, 0], i["B"][..., 0], i["C"][..., 0],
                              D=i["D"], z=i["z"], delta_bias=i["delta_bias"], h0=i["h0"][..., 0],
                              lib=lib)
    yc, lc = P.sm1_closed_form(i["x"], i["delta"], i["A"][:, 0], i["B"][..., 0], i["C"][..., 0],
                               i["h0"][..., 0], bias=i["delta_bias"])
    yc = P.ref_gate(yc + i["D"][None, None].astype(np.float64) * i["x"], i["z"].astype(np.float64))
    assert P._rel(y, yc) < 1e-11 and P._rel(last, lc) < 1e-11
