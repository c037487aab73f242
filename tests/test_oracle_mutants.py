"""Plant plausible mistakes in a copy of the oracle source (on the CPU only)
and check that the pins in oracle_pins.py catch every one of them.

The real oracle source is never modified: each mutant is a text substitution
written to a temporary file, compiled with the same flags and loaded on its
own.  A mutant "survives" when every pin still passes; that would mean the
pins could not tell that mistake from the definition.
"""
import os

import pytest

import oracle
import oracle_pins as P

SRC = os.path.join(os.path.dirname(oracle.__file__), "ssm_oracle.c")

MUTANTS = [
    ("drop D skip", "out += Dv[d] * xv;", "out += 0.0 * xv;"),
    ("decay exponent sign", "exp(dt * A[d * dstate + n])", "exp(-dt * A[d * dstate + n])"),
    ("decay without Delta", "exp(dt * A[d * dstate + n])", "exp(A[d * dstate + n])"),
    ("A transposed", "exp(dt * A[d * dstate + n])", "exp(dt * A[n * dim + d])"),
    ("B replaced by C", "dt * Bm[bt * dstate + n] * xv", "dt * Cm[bt * dstate + n] * xv"),
    ("C replaced by B", "out += Cm[bt * dstate + n] * h[n];", "out += Bm[bt * dstate + n] * h[n];"),
    ("input without Delta", "+ dt * Bm[bt * dstate + n] * xv", "+ Bm[bt * dstate + n] * xv"),
    ("B one step late", "dt * Bm[bt * dstate + n] * xv",
     "dt * Bm[(t > 0 ? bt - 1 : bt) * dstate + n] * xv"),
    ("decay applied after input", "h[n] = decay * h[n] + dt * Bm[bt * dstate + n] * xv;",
     "h[n] = decay * (h[n] + dt * Bm[bt * dstate + n] * xv);"),
    ("softplus dropped", "delta_softplus ? softplus(v) : v", "v"),
    ("softplus always on", "delta_softplus ? softplus(v) : v", "softplus(v)"),
    ("bias dropped", "v += delta_bias[d];", "v += 0.0;"),
    ("softplus negative branch", "return log1p(exp(v));", "return exp(v);"),
    ("softplus positive branch", "return v + log1p(exp(-v));", "return v;"),
    ("gate by z, not SiLU(z)", "out *= silu(z[bt * dim + d]);", "out *= z[bt * dim + d];"),
    ("SiLU sign", "return v / (1.0 + exp(-v));", "return v / (1.0 + exp(v));"),
    ("h0 ignored", "h[n] = h0 ? h0[(b * dim + d) * dstate + n] : 0.0;", "h[n] = 0.0;"),
    ("last_state not the final state", "last_state[(b * dim + d) * dstate + n] = h[n];",
     "last_state[(b * dim + d) * dstate + n] = 0.0;"),
    ("readout uses first state only", "out += Cm[bt * dstate + n] * h[n];",
     "out += Cm[bt * dstate + n] * h[0];"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site not unique for {name!r}"
    path = tmp_path / "mutant.c"
    path.write_text(src.replace(old, new))
    lib = oracle.load(oracle.build(str(path), str(tmp_path / "libmutant.so")))
    caught = []
    for pin in P.ALL_PINS:
        try:
            pin(lib)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"mutant {name!r} passed every pin"
