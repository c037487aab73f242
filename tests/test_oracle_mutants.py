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
    # the backward
    ("bwd: adjoint not decayed", "g[n] *= a;", "g[n] *= 1.0;"),
    ("bwd: dlast ignored", "g[n] = dlast ? dlast[(b * dim + d) * dstate + n] : 0.0;", "g[n] = 0.0;"),
    ("bwd: dA without Delta", "dA[d * dstate + n] += g[n] * dt * a * h_prev[n];",
     "dA[d * dstate + n] += g[n] * a * h_prev[n];"),
    ("bwd: dA with the new state", "dA[d * dstate + n] += g[n] * dt * a * h_prev[n];",
     "dA[d * dstate + n] += g[n] * dt * a * h_now[n];"),
    ("bwd: dB from the output gradient", "dB[bt * dstate + n] += g[n] * dt * xv;",
     "dB[bt * dstate + n] += dyv * dt * xv;"),
    ("bwd: dC with the previous state", "dC[bt * dstate + n] += dyv * h_now[n];",
     "dC[bt * dstate + n] += dyv * h_prev[n];"),
    ("bwd: decay term sign in dDelta", "ddt += g[n] * (A[d * dstate + n] * a * h_prev[n]",
     "ddt += g[n] * (-A[d * dstate + n] * a * h_prev[n]"),
    ("bwd: input term dropped from dDelta", "+ Bm[bt * dstate + n] * xv);", ");"),
    ("bwd: softplus derivative", "ddt * sigmoid(vs[t])", "ddt * softplus(vs[t])"),
    ("bwd: SiLU derivative sign", "(1.0 + zv * (1.0 - s))", "(1.0 - zv * (1.0 - s))"),
    ("bwd: dx misses the D skip", "double dxv = Dv ? dyv * Dv[d] : 0.0;", "double dxv = 0.0;"),
    ("bwd: dD from the ungated gradient", "dD[d] += dyv * xv;", "dD[d] += go * xv;"),
    ("bwd: dx from the state gradient uses C", "dxv += g[n] * dt * Bm[bt * dstate + n];",
     "dxv += g[n] * dt * Cm[bt * dstate + n];"),
    ("bwd: recomputed state without Delta in the input",
     "hs[(t + 1) * dstate + n] = decay * hs[t * dstate + n] + dt * Bm[bt * dstate + n] * xv;",
     "hs[(t + 1) * dstate + n] = decay * hs[t * dstate + n] + Bm[bt * dstate + n] * xv;"),
    ("bwd: step decay sign", "const double a = exp(dt * A[d * dstate + n]);",
     "const double a = exp(-dt * A[d * dstate + n]);"),
    ("bwd: softplus derivative at Delta", "vs[t] = v;", "vs[t] = dt;"),
    # the causal convolution
    ("conv: filter reversed", "acc += w[d * width + k] * v;", "acc += w[d * width + (H - k)] * v;"),
    ("conv: history one step late", "const long s = t - H + k;", "const long s = t - width + k;"),
    ("conv: bias dropped", "double acc = bias ? bias[d] : 0.0;\n            for (long k = 0; k < width; ++k)",
     "double acc = 0.0;\n            for (long k = 0; k < width; ++k)"),
    ("conv decode: bias dropped", "double acc = bias ? bias[d] : 0.0;\n        for (long k = 0; k < H; ++k)",
     "double acc = 0.0;\n        for (long k = 0; k < H; ++k)"),
    ("conv: SiLU dropped", "out[(b * seqlen + t) * dim + d] = silu_on ? silu(acc) : acc;",
     "out[(b * seqlen + t) * dim + d] = acc;"),
    ("conv: state ignored", "v = state_in ? state_in[(b * dim + d) * H + (H + s)] : 0.0;\n                acc",
     "v = 0.0;\n                acc"),
    ("conv: state_out from the start", "const long s = seqlen - H + j;", "const long s = j;"),
    ("conv decode: window not shifted", "st[k] = st[k + 1];", "st[k] = st[k];"),
    ("conv decode: newest tap on the oldest input", "acc += w[d * width + H] * x[b * dim + d];",
     "acc += w[d * width] * x[b * dim + d];"),
    # the Mamba-2 multi-head scan
    ("ssd: decay of head 0", "const double decay = exp(delta * A[h]);",
     "const double decay = exp(delta * A[0]);"),
    ("ssd: decay sign", "const double decay = exp(delta * A[h]);",
     "const double decay = exp(-delta * A[h]);"),
    ("ssd: input without Delta", "s[n] = decay * s[n] + delta * Bm[bt * dstate + n] * xv;",
     "s[n] = decay * s[n] + Bm[bt * dstate + n] * xv;"),
    ("ssd: dt of head 0", "double v = dt[bt * nheads + h];", "double v = dt[bt * nheads];"),
    ("ssd: bias of head 0", "v += dt_bias[h];", "v += dt_bias[0];"),
    ("ssd: softplus dropped", "const double delta = dt_softplus ? softplus(v) : v;",
     "const double delta = v;"),
    ("ssd: x in (B, T, P, H) order", "const long xi = (bt * nheads + h) * headdim + p;",
     "const long xi = (bt * headdim + p) * nheads + h;"),
    ("ssd: head from the wrong digit", "const long h = (c / headdim) % nheads;",
     "const long h = c % nheads;"),
    ("ssd: C replaced by B", "out += Cm[bt * dstate + n] * s[n];", "out += Bm[bt * dstate + n] * s[n];"),
    ("ssd: D of head 0", "out += Dv[h] * xv;", "out += Dv[0] * xv;"),
    ("ssd: gate by z", "out *= silu(z[xi]);", "out *= z[xi];"),
    ("ssd: h0 ignored", "s[n] = h0 ? h0[c * dstate + n] : 0.0;", "s[n] = 0.0;"),
    ("ssd: last state not final", "last_state[c * dstate + n] = s[n];", "last_state[c * dstate + n] = 0.0;"),
    # dt_proj
    ("dt_proj: W transposed", "acc += xdt[m * ldx + k] * W[d * rank + k];",
     "acc += xdt[m * ldx + k] * W[k * dim + d];"),
    ("dt_proj: row stride ignored", "acc += xdt[m * ldx + k] * W[d * rank + k];",
     "acc += xdt[m * rank + k] * W[d * rank + k];"),
    ("dt_proj: whole row read", "for (long k = 0; k < rank; ++k)\n                acc +=",
     "for (long k = 0; k < ldx; ++k)\n                acc +="),
    ("dt_proj: first column dropped", "for (long k = 0; k < rank; ++k)\n                acc +=",
     "for (long k = 1; k < rank; ++k)\n                acc +="),
    ("dt_proj: output transposed", "out[m * dim + d] = acc;", "out[d * rows + m] = acc;"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    src = open(SRC).read()
    # a statement of the forward body that the backward repeats in its own
    # forward sweep is mutated in both places: the same mistake in the definition
    assert src.count(old) >= 1, f"mutation site missing for {name!r}"
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
