"""Pins of the fp64 minGRU-cell oracle (the gate fused ahead of the log-space scan).

oracle.mingru_fwd / mingru_bwd (oracle/oracle.c) are checked against:
hand-derived worked examples (tests/golden/mingru_cell_worked.json, both
branches of g), the separately pinned log-space scan oracle applied to the
generator's own log-space gate recipe (synthetic.mingru_logs, numpy code that
shares nothing with oracle.c), the chain rule through that recipe for the
gradients, and central finite differences.
"""
import json
import os

import numpy as np

import oracle
from synthetic import mingru_inputs, mingru_logs

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rel(x, r):
    x, r = np.asarray(x, np.float64), np.asarray(r, np.float64)
    return float(np.max(np.abs(x - r)) / max(np.max(np.abs(r)), 1e-300))


def test_golden_mingru_cell():
    fx = json.load(open(os.path.join(GOLD, "mingru_cell_worked.json")))
    for case in fx["cases"]:
        col = lambda v: np.asarray(v, np.float64).reshape(1, -1, 1)
        k, x, dh = col(case["k"]), col(case["x"]), col(case["dh"])
        x0 = np.array([[case["x0"]]])
        np.testing.assert_allclose(oracle.mingru_fwd(k, x, x0).ravel(), case["h"], rtol=0, atol=1e-15)
        dk, dx, dx0 = oracle.mingru_bwd(k, x, x0, dh)
        np.testing.assert_allclose(dk.ravel(), case["dk"], rtol=0, atol=1e-15)
        np.testing.assert_allclose(dx.ravel(), case["dx"], rtol=0, atol=1e-15)
        np.testing.assert_allclose(dx0.ravel(), [case["dx0"]], rtol=0, atol=1e-15)


def test_matches_log_scan_of_the_gate_recipe():
    inp = mingru_inputs(3, 200, 8, seed=41)
    la, lb, lh0 = mingru_logs(inp.k, inp.x, inp.x0)
    assert _rel(oracle.mingru_fwd(inp.k, inp.x, inp.x0), oracle.log_fwd(la, lb, lh0)) < 1e-13


def test_gradients_match_chain_rule_through_the_recipe():
    """dk = -sigmoid(k) dlog a + sigmoid(-k) dlog b;  dx = dlog b * (log g)'(x);  dx0 = dlog h0 * (log g)'(x0)."""
    inp = mingru_inputs(3, 200, 8, seed=42)
    k, x, x0 = (v.astype(np.float64) for v in (inp.k, inp.x, inp.x0))
    la, lb, lh0 = mingru_logs(k, x, x0)
    dla, dlb, dlh0 = oracle.log_bwd(la, lb, lh0, inp.dh)
    sig = lambda u: 1.0 / (1.0 + np.exp(-u))
    dlog_g = lambda u: np.where(u >= 0, 1.0 / (np.maximum(u, 0.0) + 0.5), 1.0 - sig(u))
    dk, dx, dx0 = oracle.mingru_bwd(k, x, x0, inp.dh)
    assert _rel(dk, -sig(k) * dla + sig(-k) * dlb) < 1e-11
    assert _rel(dx, dlb * dlog_g(x)) < 1e-11
    assert _rel(dx0, dlh0 * dlog_g(x0)) < 1e-11


def test_gradients_finite_difference():
    inp = mingru_inputs(2, 6, 3, seed=43)
    k, x, x0, dh = (v.astype(np.float64) for v in (inp.k, inp.x, inp.x0, inp.dh))
    # keep every probe on one side of g's kink at 0
    x = np.where(np.abs(x) < 1e-3, 1e-3, x)
    x0 = np.where(np.abs(x0) < 1e-3, 1e-3, x0)
    loss = lambda k_, x_, x0_: float(np.sum(dh * oracle.mingru_fwd(k_, x_, x0_)))
    grads = oracle.mingru_bwd(k, x, x0, dh)
    eps = 1e-6
    for v, gv in zip((k, x, x0), grads):
        flat = v.reshape(-1)
        num = np.empty_like(flat)
        for i in range(flat.size):
            old = flat[i]
            flat[i] = old + eps
            fp = loss(k, x, x0)
            flat[i] = old - eps
            fm = loss(k, x, x0)
            flat[i] = old
            num[i] = (fp - fm) / (2 * eps)
        assert np.max(np.abs(num - gv.reshape(-1))) / max(1.0, np.max(np.abs(gv))) < 1e-7
