"""Writes hand_recurrence.json: worked examples of the selective-scan recurrence
derived by hand (no implementation of the scan is called here).

Definitions followed ("Mamba State Space Models complete guide", youngju.dev):
  section 2, Discretization (ZOH): Abar = exp(Delta * A); discrete recurrence
      h[t] = Abar h[t-1] + Bbar x[t], y[t] = C h[t];
  section 5, complete Mamba implementation: the selective_scan injects
      Delta * B * x, adds the D * x skip; MambaBlock.forward gates with SiLU(z);
      Delta = softplus(projection).
The pages print no numeric input/output pair, so each case is chosen so that
every step can be done by hand: Delta = 1 and A = -ln 2, -ln 4 make the decays
exactly 1/2 and 1/4; bias = ln(e - 1) makes softplus(0 + bias) = 1; z = ln 3
makes SiLU(z) = ln 3 * 3/4.  Run: python tests/golden/make_hand_recurrence.py
"""
import json
import math
import os

LN2, LN4, LN3 = math.log(2.0), math.log(4.0), math.log(3.0)
GATE = 0.75 * LN3  # SiLU(ln 3) = ln3 * sigmoid(ln3) = ln3 * 3/(1+3)

# plain_two_states, by hand (h0 = (4, 8), x = (2, 4, 8), D = 1/2):
#   t0: h = (1/2*4 + 1*1*2, 1/4*8 + 1*1*2) = (4, 4);      y = 4 + 0      + 1/2*2 = 5
#   t1: h = (1/2*4 + 1*1*4, 1/4*4 - 1*1*4) = (6, -3);     y = 0 - 3      + 1/2*4 = -1
#   t2: h = (1/2*6 + 2*8,   1/4*(-3) + 0)  = (19, -3/4);  y = 19 - 3/4   + 1/2*8 = 22.25
PLAIN_Y = [5.0, -1.0, 22.25]
PLAIN_H = [19.0, -0.75]

CASES = [
    {"name": "plain_two_states",
     "note": "Delta=1 (softplus off, no bias), A=(-ln2,-ln4): decays (1/2, 1/4). "
             "t0 h=(4,4) y=5; t1 h=(6,-3) y=-1; t2 h=(19,-0.75) y=22.25",
     "softplus": 0, "x": [2, 4, 8], "delta": [1, 1, 1], "bias": None, "A": [-LN2, -LN4],
     "B": [[1, 1], [1, -1], [2, 0]], "C": [[1, 0], [0, 1], [1, 1]], "D": 0.5, "z": None,
     "h0": [4, 8], "y": PLAIN_Y, "last_state": PLAIN_H},
    {"name": "softplus_bias_gate",
     "note": "delta=0, bias=ln(e-1): softplus gives Delta = ln(1 + e - 1) = 1, so the states "
             "equal plain_two_states; z = ln3 scales every output by SiLU(ln3) = 0.75 ln3",
     "softplus": 1, "x": [2, 4, 8], "delta": [0, 0, 0], "bias": math.log(math.e - 1.0),
     "A": [-LN2, -LN4], "B": [[1, 1], [1, -1], [2, 0]], "C": [[1, 0], [0, 1], [1, 1]],
     "D": 0.5, "z": [LN3, LN3, LN3], "h0": [4, 8],
     "y": [v * GATE for v in PLAIN_Y], "last_state": PLAIN_H},
    {"name": "scalar_state_decay_half",
     "note": "d_state=1, Delta=1, A=-ln2 halves the state each step; h0=8, Delta*B*x=1: "
             "h=(5, 3.5, 2.75, 2.375); y=C*h with C=(1,2,1,2)",
     "softplus": 0, "x": [1, 1, 1, 1], "delta": [1, 1, 1, 1], "bias": None, "A": [-LN2],
     "B": [[1], [1], [1], [1]], "C": [[1], [2], [1], [2]], "D": None, "z": None, "h0": [8],
     "y": [5.0, 7.0, 2.75, 4.75], "last_state": [2.375]},
]

DOC = {
    "citation": "Hand-derived worked examples of h[t] = exp(Delta*A) h[t-1] + Delta*B[t]*x[t], "
                "y[t] = (C[t].h[t] + D*x[t]) * SiLU(z[t]); definitions from 'Mamba State Space "
                "Models complete guide' (youngju.dev), section 2 (ZOH, discrete recurrence) and "
                "section 5 (selective_scan: Delta*B*x, D skip; MambaBlock: SiLU(z) gate; "
                "softplus Delta). The pages print no numeric examples.",
    "layout": "batch=1, d_inner=1; x, delta, z per t; B, C per (t, n); A per n; h0, last_state per n",
    "cases": CASES,
}

if __name__ == "__main__":
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "hand_recurrence.json")
    with open(out, "w") as f:
        json.dump(DOC, f, indent=1)
    print("wrote", out)
