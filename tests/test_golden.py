"""Stored expected values: the pages' printed figures and exact rationals.

Pages cited (by title):
  [K3-memory]  "Kimi K3 Changed the Memory Math for Agentic AI Forever"
               (hubwiz.com translation), §3, §4 (memory math), §5 (snapshots).
"""
import json
import os
from fractions import Fraction

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_state_size_reproduces_printed_memory_math():
    """The oracle's final state for one session at K3's head shape, counted in
    bf16 over the 69 KDA layers, is the 217,055,232 bytes [K3-memory] §3 prints;
    the §4/§5 cache and snapshot figures follow from it to the printed digits."""
    g = _load("pages_memory_math.json")
    H, dk, dv = g["heads"], g["key_dim"], g["value_dim"]
    rng = np.random.default_rng(0)
    T = 2
    _, sT = oracle.kda_forward(rng.standard_normal((T, H, dk)), rng.standard_normal((T, H, dk)),
                               rng.standard_normal((T, H, dv)), -np.ones((T, H, dk)),
                               np.full((T, H), 0.5))
    assert sT.shape == (1, H, dv, dk)
    state_bytes = g["kda_layers"] * sT[0].size * g["bytes_per_value_bf16"]
    assert state_bytes == g["state_bytes_per_session"]
    assert round(state_bytes / 1e9, 2) == g["state_gb_per_session"]
    per_tok_layer = g["mla_cached_values_per_token_per_layer"] * g["bytes_per_value_bf16"]
    for tokens, row in g["cache_gb"].items():
        tokens = int(tokens)
        all_mla = g["total_layers"] * tokens * per_tok_layer / 1e9
        k3 = (g["mla_layers"] * tokens * per_tok_layer + state_bytes) / 1e9
        assert round(all_mla, 2) == row["all_mla"]
        assert round(k3, 2) == row["k3"]
        assert round(100 * (1 - k3 / all_mla), 1) == row["reduction_pct"]
    s = g["snapshots"]
    assert round(s["count"] * s["gb_each"], 2) == s["gb_total"]
    assert round(g["cache_gb"]["1000000"]["k3"] + s["gb_total"], 2) == s["with_cache_gb"]
    assert round(100 * (1 - s["with_cache_gb"] / g["cache_gb"]["1000000"]["all_mla"])) == \
        s["reduction_vs_all_mla_pct"]


def test_oracle_matches_stored_exact_rationals():
    """``brute_force_exact.json`` holds exact transition-product results written by
    ``tests/golden/make_golden.py`` (oracle.forms only)."""
    doc = _load("brute_force_exact.json")
    for c in doc["cases"]:
        inp = c["inputs"]
        f = lambda rows: np.array([[float(Fraction(x)) for x in row] for row in rows])
        beta = np.array([float(Fraction(x)) for x in inp["beta"]])
        out, sT = oracle.kda_forward(f(inp["q"])[:, None], f(inp["k"])[:, None],
                                     f(inp["v"])[:, None], np.log(f(inp["alpha"]))[:, None],
                                     beta[:, None], state0=f(inp["S0"]).T[None, None])
        ref_out, ref_S = f(c["out"]), f(c["S_T"])
        assert np.abs(out[:, 0] - ref_out).max() <= 1e-13 * max(1.0, np.abs(ref_out).max())
        assert np.abs(sT[0, 0] - ref_S.T).max() <= 1e-13 * max(1.0, np.abs(ref_S).max())
