"""Pins of the fp64 oracle to facts that do not come from the oracle itself.

Each `pin_*` takes a loaded oracle library and raises AssertionError when the
oracle disagrees with the fact it checks.  They are collected as tests in
test_oracle_pins.py and re-run against deliberately broken copies of the
oracle source in test_oracle_mutants.py, which shows that each plausible
mistake (a dropped term, a wrong sign or index, a swapped operand) is caught.

Independent references used here (numpy / scipy, fp64):
  * hand-derived worked examples (tests/golden/hand_recurrence.json);
  * brute-force unrolling h_t = prod(Abar) h0 + sum_s prod(Abar) Delta_s B_s x_s
    (the solution of the discrete recurrence of the youngju.dev guide,
    section 2), with softplus from numpy.logaddexp and SiLU from
    scipy.special.expit;
  * the SM1 closed form L = cumprod(dA), h = L * (h0 + cumsum(dBx / L)),
    y = h * C ("Windows SM1 (Scalar Mamba1)" page, detailed sections),
    evaluated without the clamp and restarted every 64 steps so L cannot
    underflow;
  * the convolution-kernel identity for time-invariant parameters,
    K = (C Bbar, C Abar Bbar, C Abar^2 Bbar, ...), y = K * u (youngju.dev
    guide, section 2, "SSM as a convolution kernel"), by direct convolution
    and by FFT;
  * invariants: Delta = 0 keeps h at h0, A = 0 gives a running sum, linearity
    in (x, h0), D skip, SiLU gate, continuation from last_state, a decode step
    repeated T times equals the scan, and the inverse softplus of the dt
    initialisation (section 5 MambaBlock init; softplus(log(expm1(dt))) = dt).
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
from scipy.special import expit

import oracle
from selective_scan_ssm_amd import inputs as gen

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "hand_recurrence.json")


# ----------------------------------------------------------------- references
def ref_delta(delta, bias, softplus):
    v = delta + (0.0 if bias is None else bias)
    return np.logaddexp(0.0, v) if softplus else v


def ref_gate(y, z):
    return y if z is None else y * (z * expit(z))


def brute_force(x, delta, A, B, C, D=None, z=None, bias=None, softplus=True, h0=None):
    """O(T^2) unrolled solution of the recurrence; returns (y, last_state)."""
    x, delta, A, B, C = (np.asarray(a, np.float64) for a in (x, delta, A, B, C))
    Bt, T, Dd = x.shape
    N = A.shape[1]
    dt = ref_delta(delta, bias, softplus)                               # (Bt,T,Dd)
    abar = np.exp(dt[..., None] * A[None, None])                        # (Bt,T,Dd,N)
    inp = dt[..., None] * B[:, :, None, :] * x[..., None]               # (Bt,T,Dd,N)
    h0 = np.zeros((Bt, Dd, N)) if h0 is None else np.asarray(h0, np.float64)
    hs = np.zeros((Bt, T, Dd, N))
    for t in range(T):
        acc = np.prod(abar[:, 0:t + 1], axis=1) * h0
        for s in range(t + 1):
            acc = acc + np.prod(abar[:, s + 1:t + 1], axis=1) * inp[:, s]
        hs[:, t] = acc
    y = np.einsum("btdn,btn->btd", hs, C)
    if D is not None:
        y = y + np.asarray(D, np.float64)[None, None] * x
    y = ref_gate(y, None if z is None else np.asarray(z, np.float64))
    last = hs[:, -1] if T > 0 else h0.copy()
    return y, last


def sm1_closed_form(x, delta, A, B, C, h0, bias=None, softplus=True, chunk=64):
    """SM1 closed form (cumprod / cumsum), no clamp, restarted every `chunk`
    steps with the carried state as the next h0.  A: (Dd,), B, C: (Bt,T),
    h0: (Bt,Dd).  Returns (pre-skip, pre-gate y, last_state)."""
    x, delta = np.asarray(x, np.float64), np.asarray(delta, np.float64)
    Bt, T, Dd = x.shape
    dt = ref_delta(delta, bias, softplus)
    dA = np.exp(dt * np.asarray(A, np.float64)[None, None])
    dBx = dt * np.asarray(B, np.float64)[..., None] * x
    y = np.zeros_like(x)
    h_in = np.asarray(h0, np.float64).copy()
    for s in range(0, T, chunk):
        e = min(T, s + chunk)
        L = np.cumprod(dA[:, s:e], axis=1)
        h = L * (h_in[:, None, :] + np.cumsum(dBx[:, s:e] / L, axis=1))
        y[:, s:e] = h * np.asarray(C, np.float64)[:, s:e, None]
        h_in = h[:, -1]
    return y, h_in


def lti_kernel_output(x, dt, A, Bv, Cv, method):
    """Time-invariant case: y = K * x with K_k = sum_n C_n exp(k dt A_n) dt B_n.
    x: (T,) one channel; dt scalar; A, Bv, Cv: (N,)."""
    T = x.shape[0]
    k = np.arange(T)[:, None]
    K = (Cv[None] * np.exp(k * dt * A[None]) * dt * Bv[None]).sum(axis=1)
    if method == "direct":
        return np.convolve(K, x)[:T]
    n = 1 << int(math.ceil(math.log2(2 * T)))
    return np.fft.irfft(np.fft.rfft(K, n) * np.fft.rfft(x, n), n)[:T]


def _rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    den = max(np.abs(b).max(initial=0.0), 1e-300)
    return np.abs(a - b).max(initial=0.0) / den


def _small(seed=11, Bt=2, T=24, Dd=5, N=3, h0_kind="normal", a_kind="sm1"):
    inp = gen.make_inputs(Bt, T, Dd, N, io=gen.F32, a_kind=a_kind, h0_kind=h0_kind, seed=seed)
    return {k: (v.astype(np.float64) if isinstance(v, np.ndarray) else v) for k, v in inp.items()}


def _scan(lib, i, **over):
    kw = dict(D=i["D"], z=i["z"], delta_bias=i["delta_bias"], delta_softplus=True, h0=i["h0"])
    kw.update(over)
    return oracle.selective_scan(i["x"], i["delta"], i["A"], i["B"], i["C"], lib=lib, **kw)


# ----------------------------------------------------------------------- pins
def pin_golden(lib):
    doc = json.load(open(GOLDEN))
    for c in doc["cases"]:
        T, N = len(c["x"]), len(c["A"])
        x = np.array(c["x"], float).reshape(1, T, 1)
        dl = np.array(c["delta"], float).reshape(1, T, 1)
        A = np.array(c["A"], float).reshape(1, N)
        B = np.array(c["B"], float).reshape(1, T, N)
        C = np.array(c["C"], float).reshape(1, T, N)
        D = None if c["D"] is None else np.array([c["D"]], float)
        z = None if c["z"] is None else np.array(c["z"], float).reshape(1, T, 1)
        bias = None if c["bias"] is None else np.array([c["bias"]], float)
        h0 = np.array(c["h0"], float).reshape(1, 1, N)
        y, last = oracle.selective_scan(x, dl, A, B, C, D=D, z=z, delta_bias=bias,
                                        delta_softplus=bool(c["softplus"]), h0=h0, lib=lib)
        assert np.allclose(y.ravel(), c["y"], rtol=1e-12, atol=1e-12), (c["name"], y.ravel())
        assert np.allclose(last.ravel(), c["last_state"], rtol=1e-12, atol=1e-12), c["name"]


def pin_bruteforce_workload0(lib):
    w = gen.workload_inputs(0)
    i = {k: (v.astype(np.float64) if isinstance(v, np.ndarray) else v) for k, v in w.items()}
    y, last = _scan(lib, i)
    yb, lb = brute_force(i["x"], i["delta"], i["A"], i["B"], i["C"], i["D"], i["z"],
                         i["delta_bias"], True, i["h0"])
    assert _rel(y, yb) < 1e-12 and _rel(last, lb) < 1e-12


def pin_bruteforce_random(lib):
    """Random A per (d, n), nonzero h0, every optional input on."""
    i = _small(seed=5, Bt=2, T=20, Dd=4, N=3)
    i["A"] = -np.exp(np.random.default_rng(3).uniform(-2, 1, size=i["A"].shape))
    y, last = _scan(lib, i)
    yb, lb = brute_force(i["x"], i["delta"], i["A"], i["B"], i["C"], i["D"], i["z"],
                         i["delta_bias"], True, i["h0"])
    assert _rel(y, yb) < 1e-12 and _rel(last, lb) < 1e-12


def pin_bruteforce_no_softplus(lib):
    i = _small(seed=6, Bt=1, T=16, Dd=3, N=2)
    i["delta"] = np.abs(i["delta"]) * 0.3        # positive Delta without softplus
    y, last = _scan(lib, i, delta_softplus=False, delta_bias=None)
    yb, lb = brute_force(i["x"], i["delta"], i["A"], i["B"], i["C"], i["D"], i["z"],
                         None, False, i["h0"])
    assert _rel(y, yb) < 1e-12 and _rel(last, lb) < 1e-12


def pin_sm1_closed_form(lib):
    """N = 1 scan against the cumprod/cumsum closed form, SM1-workload
    distributions (A = -exp(U(-4,1)), h0 ~ N(0,1)), T = 512."""
    i = _small(seed=1, Bt=2, T=512, Dd=24, N=1)
    y, last = oracle.sm1_scan(i["x"], i["delta"], i["A"][:, 0], i["B"][..., 0], i["C"][..., 0],
                              delta_bias=i["delta_bias"], h0=i["h0"][..., 0], lib=lib)
    yc, lc = sm1_closed_form(i["x"], i["delta"], i["A"][:, 0], i["B"][..., 0], i["C"][..., 0],
                             i["h0"][..., 0], bias=i["delta_bias"])
    assert _rel(y, yc) < 1e-12 and _rel(last, lc) < 1e-12


def pin_nstate_is_sum_of_scalar_scans(lib):
    """Diagonal A: each state n is its own scalar recurrence, so the N-state
    output is the sum of N SM1 outputs (D skip and gate applied once)."""
    i = _small(seed=2, Bt=2, T=40, Dd=6, N=4)
    y, last = _scan(lib, i)
    acc = np.zeros_like(i["x"])
    for n in range(4):
        yn, ln = oracle.sm1_scan(i["x"], i["delta"], i["A"][:, n], i["B"][..., n], i["C"][..., n],
                                 delta_bias=i["delta_bias"], h0=i["h0"][..., n], lib=lib)
        acc += yn
        assert _rel(last[..., n], ln) < 1e-13
    ref = ref_gate(acc + i["D"][None, None] * i["x"], i["z"])
    assert _rel(y, ref) < 1e-12


def pin_delta_zero_keeps_state(lib):
    """Delta = 0 (softplus off, no bias): exp(0) = 1 and no input enters, so
    h stays h0 and y_t = C_t . h0 + D x_t before the gate."""
    i = _small(seed=3)
    i["delta"] = np.zeros_like(i["delta"])
    y, last = _scan(lib, i, delta_softplus=False, delta_bias=None, z=None)
    ref = np.einsum("bdn,btn->btd", i["h0"], i["C"]) + i["D"][None, None] * i["x"]
    assert _rel(y, ref) < 1e-14 and _rel(last, i["h0"]) == 0.0


def pin_A_zero_running_sum(lib):
    """A = 0: no decay, h_t = h0 + cumsum_s(Delta_s B_s x_s)."""
    i = _small(seed=4)
    i["A"] = np.zeros_like(i["A"])
    y, last = _scan(lib, i, D=None, z=None)
    dt = ref_delta(i["delta"], i["delta_bias"], True)
    h = i["h0"][:, None] + np.cumsum(dt[..., None] * i["B"][:, :, None, :] * i["x"][..., None], axis=1)
    assert _rel(y, np.einsum("btdn,btn->btd", h, i["C"])) < 1e-12
    assert _rel(last, h[:, -1]) < 1e-12


def pin_lti_convolution(lib):
    """Time-invariant Delta, B, C and h0 = 0: the scan equals y = K * x."""
    rng = np.random.default_rng(7)
    T, N = 96, 4
    A = -np.exp(rng.uniform(-2, 0.5, size=(1, N)))
    Bv, Cv = rng.standard_normal(N), rng.standard_normal(N)
    dt = 0.37
    x = rng.standard_normal((1, T, 1))
    y, _ = oracle.selective_scan(x, np.full((1, T, 1), dt), A, np.tile(Bv, (1, T, 1)),
                                 np.tile(Cv, (1, T, 1)), delta_softplus=False, lib=lib)
    for method in ("direct", "fft"):
        ref = lti_kernel_output(x[0, :, 0], dt, A[0], Bv, Cv, method)
        assert _rel(y[0, :, 0], ref) < 1e-10, method


def pin_skip_and_gate(lib):
    i = _small(seed=8)
    y_full, _ = _scan(lib, i)
    y_noD, _ = _scan(lib, i, D=None)
    y_plain, _ = _scan(lib, i, D=None, z=None)
    assert _rel(y_noD, ref_gate(y_plain, i["z"])) < 1e-14
    assert _rel(y_full, ref_gate(y_plain + i["D"][None, None] * i["x"], i["z"])) < 1e-14


def pin_softplus_values(lib):
    """Read Delta out of y_0 with A = 0, B = C = x = 1, h0 = 0 (y_0 = Delta)."""
    dts = np.exp(np.linspace(np.log(1e-3), np.log(1e-1), 7))
    cases = [(np.log(np.expm1(dts)), True, dts),                 # dt-init inverse
             (np.array([0.0]), True, np.array([math.log(2.0)])),  # softplus(0) = ln 2
             (np.array([40.0, 3.0]), True, np.array([40.0 + math.exp(-40.0), 3.0 + math.log1p(math.exp(-3.0))])),
             (np.array([-40.0, -3.0]), True, np.array([math.log1p(math.exp(-40.0)), math.log1p(math.exp(-3.0))])),
             (np.array([0.25, -0.5]), False, np.array([0.25, -0.5]))]
    for v, sp, expect in cases:
        Dd = v.shape[0]
        one = np.ones((1, 1, Dd))
        y, _ = oracle.selective_scan(one, np.zeros((1, 1, Dd)), np.zeros((Dd, 1)), np.ones((1, 1, 1)),
                                     np.ones((1, 1, 1)), delta_bias=v, delta_softplus=sp, lib=lib)
        assert np.allclose(y[0, 0], expect, rtol=1e-14, atol=0), (v, y[0, 0], expect)


def pin_continuation(lib):
    i = _small(seed=9, T=30)
    y, last = _scan(lib, i)
    t1 = 11
    part = {k: v for k, v in i.items()}
    ya, la = oracle.selective_scan(i["x"][:, :t1], i["delta"][:, :t1], i["A"], i["B"][:, :t1],
                                   i["C"][:, :t1], D=i["D"], z=i["z"][:, :t1],
                                   delta_bias=i["delta_bias"], h0=part["h0"], lib=lib)
    yb, lb = oracle.selective_scan(i["x"][:, t1:], i["delta"][:, t1:], i["A"], i["B"][:, t1:],
                                   i["C"][:, t1:], D=i["D"], z=i["z"][:, t1:],
                                   delta_bias=i["delta_bias"], h0=la, lib=lib)
    assert _rel(np.concatenate([ya, yb], axis=1), y) < 1e-13 and _rel(lb, last) < 1e-13


def pin_decode_steps_equal_scan(lib):
    i = _small(seed=10, T=12)
    y, last = _scan(lib, i)
    st = i["h0"]
    ys = []
    for t in range(12):
        yt, st = oracle.state_update(st, i["x"][:, t], i["delta"][:, t], i["A"], i["B"][:, t],
                                     i["C"][:, t], D=i["D"], z=i["z"][:, t],
                                     delta_bias=i["delta_bias"], lib=lib)
        ys.append(yt)
    assert _rel(np.stack(ys, axis=1), y) < 1e-13 and _rel(st, last) < 1e-13


def pin_linearity(lib):
    """For fixed Delta the pre-gate scan is linear in (x, h0) jointly."""
    i = _small(seed=12)
    j = _small(seed=13)
    a, b = 0.7, -1.3

    def run(x, h0):
        return oracle.selective_scan(x, i["delta"], i["A"], i["B"], i["C"], D=i["D"],
                                     delta_bias=i["delta_bias"], h0=h0, lib=lib)

    y1, l1 = run(i["x"], i["h0"])
    y2, l2 = run(j["x"], j["h0"])
    y3, l3 = run(a * i["x"] + b * j["x"], a * i["h0"] + b * j["h0"])
    assert _rel(y3, a * y1 + b * y2) < 1e-12 and _rel(l3, a * l1 + b * l2) < 1e-12


def pin_empty_sequence(lib):
    """T = 0: nothing is produced and last_state = h0."""
    i = _small(seed=14, T=0)
    y, last = _scan(lib, i)
    assert y.shape[1] == 0 and _rel(last, i["h0"]) == 0.0


# ------------------------------------------------------------ backward pins
# The gradient of the scan (oracle_selective_scan_bwd) is pinned to the
# forward oracle (itself pinned above) by central finite differences, to the
# adjoint identity of the linear part, and to closed forms at A = 0.

_GRAD_OF = {"x": "dx", "delta": "ddelta", "z": "dz", "B": "dB", "C": "dC", "A": "dA", "D": "dD",
            "delta_bias": "ddelta_bias", "h0": "dh0"}


def _bwd(lib, i, dout, dlast, softplus=True, **over):
    kw = dict(D=i["D"], z=i["z"], delta_bias=i["delta_bias"], delta_softplus=softplus, h0=i["h0"],
              dlast=dlast)
    kw.update(over)
    return oracle.selective_scan_bwd(i["x"], i["delta"], i["A"], i["B"], i["C"], dout, lib=lib, **kw)


def fd_gradients(lib, i, W, Wl, softplus, names, eps=1e-6):
    """Central differences of L = sum(W * y) + sum(Wl * last_state) through
    the forward oracle, one input element at a time."""
    def loss(ii):
        y, last = oracle.selective_scan(ii["x"], ii["delta"], ii["A"], ii["B"], ii["C"], D=ii["D"],
                                        z=ii["z"], delta_bias=ii["delta_bias"],
                                        delta_softplus=softplus, h0=ii["h0"], lib=lib)
        return float((W * y).sum() + (Wl * last).sum())

    out = {}
    for name in names:
        base = i[name]
        g = np.zeros_like(base)
        for idx in np.ndindex(base.shape):
            v0 = base[idx]
            h = eps * max(1.0, abs(v0))
            hi, lo = dict(i), dict(i)
            hi[name], lo[name] = base.copy(), base.copy()
            hi[name][idx], lo[name][idx] = v0 + h, v0 - h
            g[idx] = (loss(hi) - loss(lo)) / (2.0 * h)
        out[name] = g
    return out


def pin_bwd_finite_differences(lib):
    """Every gradient against central differences of the forward, with every
    optional input on (softplus, bias, D, gate, h0, dL/dlast_state), and with
    softplus, bias and gate off."""
    rng = np.random.default_rng(31)
    i = _small(seed=21, Bt=2, T=6, Dd=3, N=3)
    i["A"] = -np.exp(rng.uniform(-1.5, 0.5, size=i["A"].shape))
    W, Wl = rng.standard_normal(i["x"].shape), rng.standard_normal(i["h0"].shape)
    g = _bwd(lib, i, W, Wl)
    fd = fd_gradients(lib, i, W, Wl, True, list(_GRAD_OF))
    for name, key in _GRAD_OF.items():
        assert _rel(g[key], fd[name]) < 1e-7, (name, _rel(g[key], fd[name]))

    j = _small(seed=22, Bt=1, T=7, Dd=2, N=2)
    j["delta"] = np.abs(j["delta"]) * 0.5 + 0.05     # positive Delta without softplus
    j["z"], j["delta_bias"] = None, None
    W, Wl = rng.standard_normal(j["x"].shape), rng.standard_normal(j["h0"].shape)
    g = _bwd(lib, j, W, Wl, softplus=False)
    assert g["dz"] is None and g["ddelta_bias"] is None
    names = [n for n in _GRAD_OF if n not in ("z", "delta_bias")]
    fd = fd_gradients(lib, j, W, Wl, False, names)
    for name in names:
        assert _rel(g[_GRAD_OF[name]], fd[name]) < 1e-7, (name, _rel(g[_GRAD_OF[name]], fd[name]))


def pin_bwd_adjoint_identity(lib):
    """For fixed Delta and no gate, (x, h0) -> (y, last_state) is linear, and
    the backward applies its transpose: <dy, y> + <dl, last> = <dx, x> + <dh0, h0>."""
    rng = np.random.default_rng(32)
    i = _small(seed=23, Bt=2, T=20, Dd=4, N=3)
    y, last = _scan(lib, i, z=None)
    dy, dl = rng.standard_normal(y.shape), rng.standard_normal(last.shape)
    g = _bwd(lib, i, dy, dl, z=None)
    lhs = (dy * y).sum() + (dl * last).sum()
    rhs = (g["dx"] * i["x"]).sum() + (g["dh0"] * i["h0"]).sum()
    # x also enters through nothing else here (Delta does not depend on x)
    assert abs(lhs - rhs) <= 1e-12 * max(abs(lhs), 1.0), (lhs, rhs)


def pin_bwd_A_zero_closed_form(lib):
    """A = 0: no decay, so dL/dh_t = dlast + sum_{s >= t} C_s dy_s (a reverse
    cumulative sum), and every gradient has a closed form in it."""
    rng = np.random.default_rng(33)
    i = _small(seed=24, Bt=2, T=15, Dd=3, N=3)
    i["A"] = np.zeros_like(i["A"])
    dy, dl = rng.standard_normal(i["x"].shape), rng.standard_normal(i["h0"].shape)
    g = _bwd(lib, i, dy, dl, D=None, z=None)
    dt = ref_delta(i["delta"], i["delta_bias"], True)                          # (Bt,T,Dd)
    v = i["delta"] + i["delta_bias"][None, None]
    u = dt[..., None] * i["B"][:, :, None, :] * i["x"][..., None]             # (Bt,T,Dd,N)
    h = i["h0"][:, None] + np.cumsum(u, axis=1)                              # h_t
    h_prev = np.concatenate([i["h0"][:, None], h[:, :-1]], axis=1)          # h_{t-1}
    cdy = i["C"][:, :, None, :] * dy[..., None]                              # (Bt,T,Dd,N)
    G = dl[:, None] + np.flip(np.cumsum(np.flip(cdy, 1), axis=1), 1)         # dL/dh_t
    assert _rel(g["dh0"], G[:, 0]) < 1e-12
    assert _rel(g["dC"], np.einsum("btd,btdn->btn", dy, h)) < 1e-12
    assert _rel(g["dB"], np.einsum("btdn,btd->btn", G, dt * i["x"])) < 1e-12
    assert _rel(g["dx"], np.einsum("btdn,btn->btd", G, i["B"]) * dt) < 1e-12
    assert _rel(g["dA"], np.einsum("btdn,btd,btdn->dn", G, dt, h_prev)) < 1e-12
    ddt = np.einsum("btdn,btn->btd", G, i["B"]) * i["x"]
    assert _rel(g["ddelta"], ddt * expit(v)) < 1e-12
    assert _rel(g["ddelta_bias"], (ddt * expit(v)).sum(axis=(0, 1))) < 1e-12


# -------------------------------------------------------- causal conv1d pins
# The block's depthwise causal convolution (oracle_causal_conv1d) against
# numpy's full convolution (np.convolve), an impulse response written out by
# hand, and the decode / continuation identities.

def _conv_case(seed, Bt=2, T=37, Dd=5, K=4):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((Bt, T, Dd)), rng.standard_normal((Dd, K)),
            rng.standard_normal(Dd), rng.standard_normal((Bt, Dd, K - 1)))


def conv_reference(x, w, bias, state, silu):
    """np.convolve of each channel's history + inputs with the reversed filter."""
    Bt, T, Dd = x.shape
    K = w.shape[1]
    out = np.zeros_like(x)
    for b in range(Bt):
        for d in range(Dd):
            hist = np.zeros(K - 1) if state is None else state[b, d]
            ext = np.concatenate([hist, x[b, :, d]])
            full = np.convolve(ext, w[d, ::-1])
            out[b, :, d] = full[K - 1:K - 1 + T] + (0.0 if bias is None else bias[d])
    return out * expit(out) if silu else out


def pin_conv_numpy_convolve(lib):
    for K in (1, 2, 4):
        x, w, bias, state = _conv_case(40 + K, K=K)
        for st, sl, bi in ((None, True, bias), (state, True, bias), (state, False, None)):
            out, so = oracle.causal_conv1d(x, w, bi, st, silu=sl, lib=lib)
            assert _rel(out, conv_reference(x, w, bi, st, sl)) < 1e-14, (K, st is None, sl)
            ext = np.concatenate([np.zeros((2, 5, K - 1)) if st is None else st,
                                  np.transpose(x, (0, 2, 1))], axis=2)
            assert np.array_equal(so, ext[:, :, ext.shape[2] - (K - 1):]), K


def pin_conv_impulse_response(lib):
    """A unit impulse at step 5 of one channel returns the filter, last tap first."""
    K, T = 4, 12
    w = np.array([[0.5, -1.25, 2.0, 3.0]])
    x = np.zeros((1, T, 1))
    x[0, 5, 0] = 1.0
    out, _ = oracle.causal_conv1d(x, w, None, None, silu=False, lib=lib)
    expect = np.zeros(T)
    expect[5:9] = [3.0, 2.0, -1.25, 0.5]
    assert np.array_equal(out[0, :, 0], expect), out[0, :, 0]


def pin_conv_decode_and_continuation(lib):
    x, w, bias, state = _conv_case(47, T=20)
    out, so = oracle.causal_conv1d(x, w, bias, state, silu=True, lib=lib)
    st = state
    steps = []
    for t in range(20):
        o, st = oracle.conv1d_update(st, x[:, t], w, bias, silu=True, lib=lib)
        steps.append(o)
    assert _rel(np.stack(steps, axis=1), out) < 1e-15 and np.array_equal(st, so)
    o1, s1 = oracle.causal_conv1d(x[:, :7], w, bias, state, silu=True, lib=lib)
    o2, s2 = oracle.causal_conv1d(x[:, 7:], w, bias, s1, silu=True, lib=lib)
    assert _rel(np.concatenate([o1, o2], axis=1), out) < 1e-15 and np.array_equal(s2, so)
    # a sequence shorter than the window keeps part of the incoming state
    o3, s3 = oracle.causal_conv1d(x[:, :2], w, bias, state, silu=True, lib=lib)
    assert np.array_equal(s3, np.concatenate([state[:, :, 2:], np.transpose(x[:, :2], (0, 2, 1))], axis=2))


# --------------------------------------------------------------- 2-D scan pins
# The four visiting orders of the 2-D scan (oracle.scan_2d) against their
# definitions written another way: the reverse order as the brute-force
# recurrence run backwards in time, the column-major orders as the row-major
# ones on the transposed patch grid, and orders that coincide on 1 x W grids.

def pin_scan2d_reverse_is_backward_recurrence(lib):
    i = _small(seed=50, Bt=2, T=12, Dd=3, N=2)
    y, last = oracle.scan_2d(i["x"], i["delta"], i["A"], i["B"], i["C"], 3, 4, 1, D=i["D"], z=i["z"],
                             delta_bias=i["delta_bias"], h0=i["h0"], lib=lib)
    rev = lambda a: None if a is None else a[:, ::-1]
    yb, lb = brute_force(rev(i["x"]), rev(i["delta"]), i["A"], rev(i["B"]), rev(i["C"]), i["D"],
                         rev(i["z"]), i["delta_bias"], True, i["h0"])
    assert _rel(y, yb[:, ::-1]) < 1e-12 and _rel(last, lb) < 1e-12


def pin_scan2d_column_major_is_transposed_grid(lib):
    H, W = 3, 5
    i = _small(seed=51, Bt=1, T=H * W, Dd=2, N=3)
    grid_t = lambda a: None if a is None else np.ascontiguousarray(
        a.reshape(a.shape[0], H, W, -1).transpose(0, 2, 1, 3).reshape(a.shape[0], H * W, -1))
    for direction in (2, 3):
        y, last = oracle.scan_2d(i["x"], i["delta"], i["A"], i["B"], i["C"], H, W, direction, D=i["D"],
                                 z=i["z"], delta_bias=i["delta_bias"], h0=i["h0"], lib=lib)
        yt, lt = oracle.scan_2d(grid_t(i["x"]), grid_t(i["delta"]), i["A"], grid_t(i["B"]), grid_t(i["C"]),
                                W, H, direction - 2, D=i["D"], z=grid_t(i["z"]),
                                delta_bias=i["delta_bias"], h0=i["h0"], lib=lib)
        # yt is in the transposed grid's row-major order: transpose back
        back = yt.reshape(1, W, H, -1).transpose(0, 2, 1, 3).reshape(1, H * W, -1)
        assert _rel(y, back) < 1e-14 and _rel(last, lt) < 1e-14, direction


def pin_scan2d_degenerate_grids(lib):
    i = _small(seed=52, Bt=2, T=7, Dd=3, N=2)
    y0, l0 = _scan(lib, i)
    a = dict(D=i["D"], z=i["z"], delta_bias=i["delta_bias"], h0=i["h0"], lib=lib)
    args = (i["x"], i["delta"], i["A"], i["B"], i["C"])
    for H, W, direction in ((1, 7, 0), (7, 1, 0), (7, 1, 2), (1, 7, 2)):   # a line: all the same order
        y, last = oracle.scan_2d(*args, H, W, direction, **a)
        assert np.array_equal(y, y0) and np.array_equal(last, l0), (H, W, direction)
    # and the two reversed orders of a line agree
    y1, l1 = oracle.scan_2d(*args, 1, 7, 1, **a)
    y3, l3 = oracle.scan_2d(*args, 7, 1, 3, **a)
    assert np.array_equal(y1, y3) and np.array_equal(l1, l3)


# The Mamba-2 multi-head scan (oracle.ssd_scan) against its duality form and
# the Mamba-1 scan it specialises (youngju.dev guide, section 6 "Mamba 2":
# the SSM with a scalar decay per head is a semiseparable matrix acting on
# the sequence, i.e. a masked attention-like product).

def _ssd_small(seed=60, Bt=2, T=19, H=3, P=4, N=5, h0_kind="normal", **kw):
    i = gen.make_ssd_inputs(Bt, T, H, P, N, io=gen.F32, h0_kind=h0_kind, seed=seed, **kw)
    return {k: (v.astype(np.float64) if isinstance(v, np.ndarray) else v) for k, v in i.items()}


def _ssd(lib, i, **over):
    kw = dict(D=i["D"], z=i["z"], dt_bias=i["dt_bias"], dt_softplus=True, h0=i["h0"])
    kw.update(over)
    return oracle.ssd_scan(i["x"], i["dt"], i["A"], i["B"], i["C"], lib=lib, **kw)


def ssd_matrix_form(x, dt, A, B, C, D=None, z=None, bias=None, softplus=True, h0=None):
    """y = M x per (batch, head) with the lower-triangular semiseparable matrix
    M[t, s] = (C_t . B_s) Delta_s exp(sum_{s<r<=t} Delta_r A_h), plus the decayed
    initial state read out by C; last state likewise.  Exponent sums are taken
    term by term (no cumulative-sum differences)."""
    x, dt, B, C = (np.asarray(a, np.float64) for a in (x, dt, B, C))
    Bt, T, H, P = x.shape
    N = B.shape[2]
    delta = ref_delta(dt, bias, softplus)                                 # (Bt,T,H)
    y = np.zeros((Bt, T, H, P))
    last = np.zeros((Bt, H, P, N))
    for b in range(Bt):
        G = C[b] @ B[b].T                                                 # (T,T): C_t . B_s
        for h in range(H):
            a = delta[b, :, h] * A[h]
            E = np.zeros((T + 1, T + 1))                                  # E[t,s] = sum_{s<r<=t} a_r
            for t in range(T):
                for s_ in range(t + 1):
                    E[t, s_] = sum(a[r] for r in range(s_ + 1, t + 1))
            M = np.zeros((T, T))
            for t in range(T):
                for s_ in range(t + 1):
                    M[t, s_] = G[t, s_] * delta[b, s_, h] * math.exp(E[t, s_])
            yh = M @ x[b, :, h, :]                                        # (T,P)
            to_end = np.array([math.exp(sum(a[r] for r in range(s_ + 1, T))) for s_ in range(T)])
            lh = (x[b, :, h, :] * (delta[b, :, h] * to_end)[:, None]).T @ B[b]   # (P,N)
            if h0 is not None:
                dec = np.array([math.exp(sum(a[r] for r in range(t + 1))) for t in range(T)])
                yh = yh + (C[b] * dec[:, None]) @ np.asarray(h0[b, h], np.float64).T
                lh = lh + math.exp(float(np.sum(a))) * np.asarray(h0[b, h], np.float64)
            if D is not None:
                yh = yh + D[h] * x[b, :, h, :]
            y[b, :, h, :] = ref_gate(yh, None if z is None else np.asarray(z, np.float64)[b, :, h, :])
            last[b, h] = lh
    return y, last


def pin_ssd_semiseparable_matrix_form(lib):
    i = _ssd_small()
    y, last = _ssd(lib, i)
    ym, lm = ssd_matrix_form(i["x"], i["dt"], i["A"], i["B"], i["C"], i["D"], i["z"], i["dt_bias"],
                             True, i["h0"])
    assert _rel(y, ym) < 1e-12 and _rel(last, lm) < 1e-12
    # no options: no gate, skip, bias, softplus or initial state
    j = _ssd_small(seed=61, T=13, H=2, P=3, N=4, h0_kind="none", with_z=False, with_D=False,
                   with_bias=False)
    j["dt"] = np.abs(j["dt"]) * 0.3
    y, last = _ssd(lib, j, dt_softplus=False)
    ym, lm = ssd_matrix_form(j["x"], j["dt"], j["A"], j["B"], j["C"], softplus=False)
    assert _rel(y, ym) < 1e-12 and _rel(last, lm) < 1e-12


def pin_ssd_is_mamba1_with_tied_decay(lib):
    """P channels of head h scanned by the Mamba-1 scan with A[d, n] = A_h,
    Delta[d] = Delta_h, D[d] = D_h for every one of the head's channels."""
    i = _ssd_small(seed=62, T=23, H=3, P=4, N=3)
    Bt, T, H, P, N = 2, 23, 3, 4, 3
    rep = lambda v: np.repeat(np.asarray(v, np.float64), P, axis=-1)
    y1, l1 = oracle.selective_scan(i["x"].reshape(Bt, T, H * P), rep(i["dt"]),
                                   np.repeat(i["A"], P)[:, None] * np.ones((1, N)), i["B"], i["C"],
                                   D=rep(i["D"]), z=i["z"].reshape(Bt, T, H * P),
                                   delta_bias=rep(i["dt_bias"]), h0=i["h0"].reshape(Bt, H * P, N), lib=lib)
    y, last = _ssd(lib, i)
    assert _rel(y, y1.reshape(y.shape)) < 1e-14 and _rel(last, l1.reshape(last.shape)) < 1e-14


def pin_ssd_A_zero_running_sum(lib):
    i = _ssd_small(seed=63, T=17, H=2, P=3, N=4)
    i["A"] = np.zeros_like(i["A"])
    y, last = _ssd(lib, i, D=None, z=None)
    delta = ref_delta(i["dt"], i["dt_bias"], True)                        # (Bt,T,H)
    inc = delta[..., None, None] * i["x"][..., None] * i["B"][:, :, None, None, :]   # (Bt,T,H,P,N)
    s = i["h0"][:, None] + np.cumsum(inc, axis=1)
    assert _rel(y, np.einsum("btn,bthpn->bthp", i["C"], s)) < 1e-12
    assert _rel(last, s[:, -1]) < 1e-12


def pin_ssd_delta_zero_keeps_state(lib):
    i = _ssd_small(seed=64, T=9, H=2, P=3, N=4)
    i["dt"] = np.zeros_like(i["dt"])
    y, last = _ssd(lib, i, dt_bias=None, dt_softplus=False)
    assert np.array_equal(last, i["h0"])
    ref = np.einsum("btn,bhpn->bthp", i["C"], i["h0"]) + i["D"][None, None, :, None] * i["x"]
    assert _rel(y, ref_gate(ref, i["z"])) < 1e-13


def pin_ssd_continuation(lib):
    i = _ssd_small(seed=65, T=21, H=2, P=3, N=4)
    y, last = _ssd(lib, i)
    cut = lambda a, sl: None if a is None else a[:, sl]
    a, b = slice(0, 8), slice(8, None)
    j = dict(i, x=cut(i["x"], a), dt=cut(i["dt"], a), z=cut(i["z"], a), B=cut(i["B"], a), C=cut(i["C"], a))
    y1, l1 = _ssd(lib, j)
    k = dict(i, x=cut(i["x"], b), dt=cut(i["dt"], b), z=cut(i["z"], b), B=cut(i["B"], b), C=cut(i["C"], b),
             h0=l1)
    y2, l2 = _ssd(lib, k)
    assert _rel(np.concatenate([y1, y2], axis=1), y) < 1e-13 and _rel(l2, last) < 1e-13


# ------------------------------------------------------------------ dt_proj
# delta = xdt[:, :rank] @ W.T (youngju.dev guide, section 5 MambaBlock: the
# dt_proj linear layer; its bias is the scan's delta_bias).

def pin_dt_proj_unit_rows(lib):
    """Row k of the identity picks column k of W.  The columns past `rank` of
    each row hold NaN, so reading any of them would show."""
    rank, D = 5, 7
    W = np.arange(D * rank, dtype=np.float64).reshape(D, rank) * 0.25 - 3.0
    xdt = np.full((rank, rank + 3), np.nan)
    xdt[:, :rank] = np.eye(rank)
    out = oracle.dt_proj(xdt, W, lib=lib)
    assert np.array_equal(out, W.T), out


def pin_dt_proj_integer_brute_force(lib):
    """Small integers: every product and sum is exact in fp64, so the result
    must equal the integer sum written out with Python ints."""
    rng = np.random.default_rng(77)
    M, rank, D, ldx = 4, 6, 3, 9
    xi = rng.integers(-4, 5, size=(M, ldx))
    Wi = rng.integers(-4, 5, size=(D, rank))
    expect = [[sum(int(xi[m, k]) * int(Wi[d, k]) for k in range(rank)) for d in range(D)] for m in range(M)]
    out = oracle.dt_proj(xi.astype(np.float64), Wi.astype(np.float64), lib=lib)
    assert np.array_equal(out, np.array(expect, dtype=np.float64)), (out, expect)


def pin_dt_proj_rank_one(lib):
    """W = u v^T: every output row is u times the scalar v . x_m."""
    rng = np.random.default_rng(78)
    M, rank, D = 6, 8, 11
    u, v = rng.standard_normal(D), rng.standard_normal(rank)
    xdt = rng.standard_normal((M, rank + 2))
    out = oracle.dt_proj(xdt, np.outer(u, v), lib=lib)
    expect = np.outer(xdt[:, :rank] @ v, u)
    assert _rel(out, expect) < 1e-13, _rel(out, expect)


def pin_dt_proj_linearity(lib):
    """Linear in its input rows: f(a x1 + b x2) = a f(x1) + b f(x2)."""
    rng = np.random.default_rng(79)
    M, rank, D = 5, 7, 9
    W = rng.standard_normal((D, rank))
    x1, x2 = rng.standard_normal((M, rank)), rng.standard_normal((M, rank))
    lhs = oracle.dt_proj(2.0 * x1 - 0.5 * x2, W, lib=lib)
    rhs = 2.0 * oracle.dt_proj(x1, W, lib=lib) - 0.5 * oracle.dt_proj(x2, W, lib=lib)
    assert _rel(lhs, rhs) < 1e-13


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
