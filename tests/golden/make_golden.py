"""Writes ``brute_force_exact.json``: exact rational KDA outputs for two tiny
dyadic inputs, computed only by ``oracle.forms.brute_force_exact`` (transition
products, no recurrence).  Run from the repository root:

    python tests/golden/make_golden.py
"""
import json
import os
import sys
from fractions import Fraction

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))
from oracle import forms  # noqa: E402

DY = [Fraction(x, 4) for x in (-4, -3, -2, -1, 0, 1, 2, 3, 4)]
ALPHA = [Fraction(1, 2), Fraction(3, 4), Fraction(7, 8), Fraction(1)]
BETA = [Fraction(1, 4), Fraction(1, 2), Fraction(3, 4), Fraction(1)]


def case(seed, T, dk, dv):
    r = np.random.default_rng(seed)
    pick = lambda pool, shape: [[pool[i] for i in row] for row in r.integers(0, len(pool), shape)]
    inp = dict(q=pick(DY, (T, dk)), k=pick(DY, (T, dk)), v=pick(DY, (T, dv)),
               alpha=pick(ALPHA, (T, dk)),
               beta=[BETA[i] for i in r.integers(0, len(BETA), T)],
               S0=pick(DY, (dk, dv)))
    out, S_T = forms.brute_force_exact(**inp)
    s = lambda x: str(x)
    enc = lambda rows: [[s(x) for x in row] for row in rows]
    return {"seed": seed, "T": T, "d_k": dk, "d_v": dv,
            "inputs": {key: (enc(val) if key != "beta" else [s(x) for x in val])
                       for key, val in inp.items()},
            "out": enc(out), "S_T": enc(S_T)}


if __name__ == "__main__":
    doc = {"what": "exact rational KDA forward (math orientation S in R^{d_k x d_v}); "
                   "alpha is the decay itself, S0 and S_T are [d_k][d_v]",
           "written_by": "tests/golden/make_golden.py via oracle.forms.brute_force_exact",
           "cases": [case(100, 8, 3, 4), case(101, 8, 4, 4)]}
    with open(os.path.join(HERE, "brute_force_exact.json"), "w") as f:
        json.dump(doc, f, indent=1)
