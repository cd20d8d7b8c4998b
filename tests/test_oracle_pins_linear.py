"""Pins of the fp64 linear-space (signed-gate) scan oracle.

oracle.linear_fwd / linear_bwd (oracle/oracle.c) are checked against facts that
do not come from them: hand-derived worked examples with negative and zero
gates (tests/golden/linear_scan_worked.json), the geometric-series closed form
for constant coefficients of either sign, numpy's cumsum and cumprod for the
special cases a = 1 and b = 0, explicit products for every term of the
unrolled recurrence, central finite differences for all three gradients, and
exact identities at full size (h is linear in (b, h0); da_t = db_t h_{t-1}).
"""
import json
import os

import numpy as np
import pytest

import oracle
from synthetic import linear_inputs

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rel(x, r):
    x, r = np.asarray(x, np.float64), np.asarray(r, np.float64)
    return float(np.max(np.abs(x - r)) / max(np.max(np.abs(r)), 1e-300))


def _col(v):
    return np.asarray(v, np.float64).reshape(1, -1, 1)


def test_golden_linear_scan():
    fx = json.load(open(os.path.join(GOLD, "linear_scan_worked.json")))
    for case in fx["cases"]:
        a, b, dh = _col(case["a"]), _col(case["b"]), _col(case["dh"])
        h0 = np.array([[case["h0"]]])
        np.testing.assert_allclose(oracle.linear_fwd(a, b, h0).ravel(), case["h"], rtol=0, atol=1e-15)
        da, db, dh0 = oracle.linear_bwd(a, b, h0, dh)
        np.testing.assert_allclose(da.ravel(), case["da"], rtol=0, atol=1e-15)
        np.testing.assert_allclose(db.ravel(), case["db"], rtol=0, atol=1e-15)
        np.testing.assert_allclose(dh0.ravel(), [case["dh0"]], rtol=0, atol=1e-15)


@pytest.mark.parametrize("a,b,h0", [(0.7, 0.3, 2.0), (-0.8, 1.5, -1.0), (-1.2, 0.4, 0.5), (-1.0, 2.0, 3.0)])
def test_constant_coefficients_geometric(a, b, h0):
    T = 30
    h = oracle.linear_fwd(np.full((1, T, 1), a), np.full((1, T, 1), b), np.array([[h0]])).ravel()
    t = np.arange(1, T + 1, dtype=np.float64)
    # h_t = a^t h0 + b (1 - a^t) / (1 - a)
    ref = a ** t * h0 + b * (1 - a ** t) / (1 - a)
    assert _rel(h, ref) < 1e-13


def test_unit_gate_is_cumsum():
    inp = linear_inputs(3, 50, 4, seed=31)
    a = np.ones_like(inp.a, dtype=np.float64)
    h = oracle.linear_fwd(a, inp.b, inp.h0)
    ref = inp.h0.astype(np.float64)[:, None, :] + np.cumsum(inp.b.astype(np.float64), axis=1)
    assert _rel(h, ref) < 1e-14


def test_zero_input_is_cumprod():
    inp = linear_inputs(3, 50, 4, seed=32)
    h = oracle.linear_fwd(inp.a, np.zeros_like(inp.b), inp.h0)
    ref = inp.h0.astype(np.float64)[:, None, :] * np.cumprod(inp.a.astype(np.float64), axis=1)
    assert _rel(h, ref) < 1e-14


def test_brute_force_products():
    """h_t = (a_t..a_1) h0 + sum_s (a_t..a_{s+1}) b_s, every product formed explicitly."""
    inp = linear_inputs(2, 9, 3, seed=33)
    a, b, h0 = (x.astype(np.float64) for x in (inp.a, inp.b, inp.h0))
    h = oracle.linear_fwd(a, b, h0)
    B, T, d = a.shape
    ref = np.empty_like(h)
    for bi in range(B):
        for c in range(d):
            for t in range(T):
                acc = np.prod(a[bi, :t + 1, c]) * h0[bi, c]
                for s in range(t + 1):
                    acc += np.prod(a[bi, s + 1:t + 1, c]) * b[bi, s, c]
                ref[bi, t, c] = acc
    assert _rel(h, ref) < 1e-13


def test_positive_gates_match_log_space_oracle():
    """For a, b, h0 > 0 the linear scan is the log-space scan of log a, log b, log h0."""
    rng = np.random.default_rng(34)
    a = rng.uniform(0.1, 1.2, (2, 40, 3))
    b = rng.uniform(0.1, 2.0, (2, 40, 3))
    h0 = rng.uniform(0.1, 2.0, (2, 3))
    dh = rng.standard_normal((2, 40, 3))
    assert _rel(oracle.linear_fwd(a, b, h0), oracle.log_fwd(np.log(a), np.log(b), np.log(h0))) < 1e-13
    da, db, dh0 = oracle.linear_bwd(a, b, h0, dh)
    dla, dlb, dlh0 = oracle.log_bwd(np.log(a), np.log(b), np.log(h0), dh)
    assert _rel(da * a, dla) < 1e-12 and _rel(db * b, dlb) < 1e-12 and _rel(dh0 * h0, dlh0) < 1e-12


def _fd_check(f, grads, inputs, eps=1e-6, tol=1e-7):
    for idx, (x, gx) in enumerate(zip(inputs, grads)):
        flat = x.reshape(-1)
        num = np.empty_like(flat)
        for i in range(flat.size):
            old = flat[i]
            flat[i] = old + eps
            fp = f(*inputs)
            flat[i] = old - eps
            fm = f(*inputs)
            flat[i] = old
            num[i] = (fp - fm) / (2 * eps)
        err = np.max(np.abs(num - gx.reshape(-1))) / max(1.0, np.max(np.abs(gx)))
        assert err < tol, (idx, err)


def test_gradients_finite_difference():
    inp = linear_inputs(2, 7, 3, seed=35)
    a, b, h0, dh = (x.astype(np.float64) for x in (inp.a, inp.b, inp.h0, inp.dh))
    loss = lambda a_, b_, h0_: float(np.sum(dh * oracle.linear_fwd(a_, b_, h0_)))
    _fd_check(loss, oracle.linear_bwd(a, b, h0, dh), [a, b, h0])


def test_invariants_full_size():
    """At the long-T shape: L = <db, b> + <dh0, h0> (h is linear in (b, h0)), da_t = db_t h_{t-1}."""
    inp = linear_inputs(16, 1024, 64, seed=36)
    a, b, h0, dh = (x.astype(np.float64) for x in (inp.a, inp.b, inp.h0, inp.dh))
    h = oracle.linear_fwd(a, b, h0)
    da, db, dh0 = oracle.linear_bwd(a, b, h0, dh)
    L = np.sum(dh * h)
    assert abs(np.sum(db * b) + np.sum(dh0 * h0) - L) <= 1e-10 * max(1.0, np.sum(np.abs(dh * h)))
    hprev = np.concatenate([h0[:, None, :], h[:, :-1, :]], axis=1)
    assert _rel(da, db * hprev) < 1e-14


def test_directional_derivative_full_size():
    inp = linear_inputs(16, 1024, 64, seed=37)
    a, b, h0, dh = (x.astype(np.float64) for x in (inp.a, inp.b, inp.h0, inp.dh))
    rng = np.random.default_rng(38)
    va, vb, v0 = rng.standard_normal(a.shape), rng.standard_normal(b.shape), rng.standard_normal(h0.shape)
    eps = 1e-6
    L = lambda s: np.sum(dh * oracle.linear_fwd(a + s * va, b + s * vb, h0 + s * v0))
    num = (L(eps) - L(-eps)) / (2 * eps)
    da, db, dh0 = oracle.linear_bwd(a, b, h0, dh)
    ana = np.sum(da * va) + np.sum(db * vb) + np.sum(dh0 * v0)
    assert abs(num - ana) <= 1e-6 * max(1.0, abs(ana))


def test_sequence_continuation():
    inp = linear_inputs(2, 40, 5, seed=39)
    full = oracle.linear_fwd(inp.a, inp.b, inp.h0)
    first = oracle.linear_fwd(inp.a[:, :17], inp.b[:, :17], inp.h0)
    rest = oracle.linear_fwd(inp.a[:, 17:], inp.b[:, 17:], first[:, -1])
    assert _rel(np.concatenate([first, rest], axis=1), full) < 1e-14
