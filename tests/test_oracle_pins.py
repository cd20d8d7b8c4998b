"""Pins of the fp64 oracle against facts that do not come from the oracle.

Each test checks the oracle (oracle/oracle.c through oracle/__init__.py)
against something independent of it: hand-derived worked examples
(tests/golden/), closed forms (geometric series), special cases that reduce to
numpy routines (cumsum, logaddexp.accumulate, multi_dot, matrix_power),
invariants (norm preservation, homogeneity), brute-force products, and
central finite differences.  A plausible slip in the oracle (a dropped term, a
wrong sign or index, a transposed operand, an off-by-one in t) breaks at least
one of them; tests/test_oracle_mutants.py checks that claim by compiling
deliberately broken copies of the oracle.
"""
import json
import os

import numpy as np
import pytest

import oracle
from synthetic import block_inputs, givens_mesh, log_inputs

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rel(x, r):
    x, r = np.asarray(x, np.float64), np.asarray(r, np.float64)
    return float(np.max(np.abs(x - r)) / max(np.max(np.abs(r)), 1e-300))


# ----------------------------------------------------------------- golden

def test_golden_log_scan():
    fx = json.load(open(os.path.join(GOLD, "log_scan_worked.json")))
    for case in fx["cases"]:
        a, b = np.array(case["a"]), np.array(case["b"])
        T = len(a)
        with np.errstate(divide="ignore"):
            la = np.log(a).reshape(1, T, 1)
            lb = np.log(b).reshape(1, T, 1)
            lh0 = np.log(np.array([[case["h0"]]]))
        dh = np.array(case["dh"]).reshape(1, T, 1)
        h = oracle.log_fwd(la, lb, lh0)
        np.testing.assert_allclose(h.ravel(), case["h"], rtol=1e-14, atol=0)
        dla, dlb, dlh0 = oracle.log_bwd(la, lb, lh0, dh)
        np.testing.assert_allclose(dla.ravel(), case["dlog_a"], rtol=1e-14, atol=1e-15)
        np.testing.assert_allclose(dlb.ravel(), case["dlog_b"], rtol=1e-14, atol=1e-15)
        np.testing.assert_allclose(dlh0.ravel(), [case["dlog_h0"]], rtol=1e-14, atol=1e-15)


def test_golden_block_affine():
    fx = json.load(open(os.path.join(GOLD, "block_scan_worked.json")))["affine"]
    A = np.array(fx["A"])[None, :, None]          # (1,T,1,2,2)
    b = np.array(fx["b"])[None]                   # (1,T,2)
    h0 = np.array(fx["h0"])[None]
    dh = np.array(fx["dh"])[None]
    h = oracle.block_affine_fwd(A, b, h0, 2)
    np.testing.assert_allclose(h[0], fx["h"], rtol=0, atol=1e-15)
    dA, db, dh0 = oracle.block_affine_bwd(A, b, h0, dh, 2)
    np.testing.assert_allclose(dA[0, :, 0], fx["dA"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(db[0], fx["db"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(dh0[0], fx["dh0"], rtol=0, atol=1e-15)


def test_golden_block_cumprod():
    fx = json.load(open(os.path.join(GOLD, "block_scan_worked.json")))["cumprod"]
    A = np.array(fx["A"])[None, :, None]
    dP = np.array(fx["dP"])[None, :, None]
    P = oracle.block_matrix_fwd(A, 2)
    np.testing.assert_allclose(P[0, :, 0], fx["P"], rtol=0, atol=1e-15)
    dA = oracle.block_matrix_bwd(A, dP, 2)
    np.testing.assert_allclose(dA[0, :, 0], fx["dA"], rtol=0, atol=1e-15)


# ------------------------------------------------- P1 closed forms (geometric)

@pytest.mark.parametrize("a,b,h0", [(0.7, 0.3, 2.0), (1.3, 0.5, 0.25), (0.05, 3.0, 1.0)])
def test_log_constant_coefficients_geometric(a, b, h0):
    T = 40
    la = np.full((1, T, 1), np.log(a))
    lb = np.full((1, T, 1), np.log(b))
    lh0 = np.full((1, 1), np.log(h0))
    t = np.arange(1, T + 1)
    expect = a ** t * h0 + b * (1 - a ** t) / (1 - a)
    h = oracle.log_fwd(la, lb, lh0)
    assert _rel(h.ravel(), expect) < 1e-13


def test_block_constant_coefficients_geometric():
    rng = np.random.default_rng(11)
    k, T = 4, 30
    M = rng.standard_normal((k, k))
    M *= 0.8 / max(abs(np.linalg.eigvals(M)))    # spectral radius 0.8, non-symmetric
    bvec = rng.standard_normal(k)
    h0 = rng.standard_normal(k)
    A = np.broadcast_to(M, (1, T, 1, k, k)).copy()
    b = np.broadcast_to(bvec, (1, T, k)).copy()
    h = oracle.block_affine_fwd(A, b, h0[None], k)
    I = np.eye(k)
    for t in range(1, T + 1):
        At = np.linalg.matrix_power(M, t)
        expect = At @ h0 + np.linalg.solve(I - M, (I - At) @ bvec)
        assert _rel(h[0, t - 1], expect) < 1e-12
    P = oracle.block_matrix_fwd(A, k)
    for t in (1, 2, 7, T):
        assert _rel(P[0, t - 1, 0], np.linalg.matrix_power(M, t)) < 1e-12


# ------------------------------- P2 special cases reducing to numpy routines

def test_log_unit_gate_is_cumsum():
    inp = log_inputs(3, 50, 5, seed=3)
    la = np.zeros_like(inp.log_a, dtype=np.float64)
    h = oracle.log_fwd(la, inp.log_b, inp.log_h0)
    expect = np.exp(inp.log_h0.astype(np.float64))[:, None, :] + np.cumsum(np.exp(inp.log_b.astype(np.float64)), axis=1)
    assert _rel(h, expect) < 1e-13


def test_log_zero_input_is_cumprod():
    inp = log_inputs(3, 50, 5, seed=4)
    lb = np.full(inp.log_b.shape, -np.inf)
    h = oracle.log_fwd(inp.log_a, lb, inp.log_h0)
    expect = np.exp(inp.log_h0.astype(np.float64)[:, None, :] + np.cumsum(inp.log_a.astype(np.float64), axis=1))
    assert _rel(h, expect) < 1e-13


def test_block_k1_equals_log_scan():
    inp = log_inputs(2, 33, 6, seed=5)
    A = np.exp(inp.log_a.astype(np.float64))[..., None, None]     # (B,T,d,1,1)
    b = np.exp(inp.log_b.astype(np.float64))
    h0 = np.exp(inp.log_h0.astype(np.float64))
    h_block = oracle.block_affine_fwd(A, b, h0, 1)
    h_log = oracle.log_fwd(inp.log_a, inp.log_b, inp.log_h0)
    assert _rel(h_block, h_log) < 1e-14
    dA, db, dh0 = oracle.block_affine_bwd(A, b, h0, inp.dh, 1)
    dla, dlb, dlh0 = oracle.log_bwd(inp.log_a, inp.log_b, inp.log_h0, inp.dh)
    # d/dlog a = a * d/da, d/dlog b = b * d/db, d/dlog h0 = h0 * d/dh0
    assert _rel(dA[..., 0, 0] * A[..., 0, 0], dla) < 1e-13
    assert _rel(db * b, dlb) < 1e-13
    assert _rel(dh0 * h0, dlh0) < 1e-13


# --------------------------------------- P3 Heinsen's log form vs the loop

def test_log_matches_heinsen_logcumsumexp():
    inp = log_inputs(4, 64, 8, seed=6)
    la = inp.log_a.astype(np.float64)
    lb = inp.log_b.astype(np.float64)
    lh0 = inp.log_h0.astype(np.float64)
    astar = np.cumsum(la, axis=1)                                  # a*_t
    terms = np.concatenate([lh0[:, None, :], lb - astar], axis=1)  # log h0, log b_t - a*_t
    lcse = np.logaddexp.accumulate(terms, axis=1)[:, 1:, :]
    expect = np.exp(astar + lcse)
    assert _rel(oracle.log_fwd(la, lb, lh0), expect) < 1e-12


# -------------------------------------------- P4 brute-force matrix products

def _chain(mats):
    return mats[0] if len(mats) == 1 else np.linalg.multi_dot(mats)


def test_block_affine_brute_force_products():
    inp = block_inputs(2, 12, 8, k=4, seed=7, h0="normal")
    A = inp.A.astype(np.float64)
    b = inp.b.astype(np.float64)
    h0 = inp.h0.astype(np.float64)
    h = oracle.block_affine_fwd(A, b, h0, 4)
    for bi in range(2):
        for j in range(2):
            sl = slice(4 * j, 4 * j + 4)
            for t in range(12):
                # h_t = (A_t..A_1) h0 + sum_s (A_t..A_{s+1}) b_s   (t, s 0-based here)
                acc = _chain([A[bi, u, j] for u in range(t, -1, -1)]) @ h0[bi, sl]
                for s in range(t + 1):
                    prod = np.eye(4) if s == t else _chain([A[bi, u, j] for u in range(t, s, -1)])
                    acc = acc + prod @ b[bi, s, sl]
                assert _rel(h[bi, t, sl], acc) < 1e-12


def test_block_cumprod_brute_force_products():
    inp = block_inputs(2, 10, 16, k=8, seed=8)
    A = inp.A.astype(np.float64)
    P = oracle.block_matrix_fwd(A, 8)
    for bi in range(2):
        for j in range(2):
            for t in range(10):
                expect = _chain([A[bi, u, j] for u in range(t, -1, -1)])
                assert _rel(P[bi, t, j], expect) < 1e-12


# ----------------------- P5 associativity: any chunking gives the same result

def _log_combine(x, y):
    # (LA1, LH1) then (LA2, LH2):  h -> a2 (a1 h + b1) + b2 in log space
    la1, lh1 = x
    la2, lh2 = y
    return la1 + la2, np.logaddexp(la2 + lh1, lh2)


def _random_bracket_reduce(items, combine, rng):
    items = list(items)
    while len(items) > 1:
        i = int(rng.integers(0, len(items) - 1))
        items[i:i + 2] = [combine(items[i], items[i + 1])]
    return items[0]


def test_log_pair_operator_any_bracketing():
    rng = np.random.default_rng(9)
    inp = log_inputs(1, 40, 3, seed=9)
    la = inp.log_a[0].astype(np.float64)
    lb = inp.log_b[0].astype(np.float64)
    lh0 = inp.log_h0[0].astype(np.float64)
    h = oracle.log_fwd(la[None], lb[None], lh0[None])[0]
    for t in (0, 1, 17, 39):
        for _ in range(5):
            LA, LH = _random_bracket_reduce([(la[s], lb[s]) for s in range(t + 1)], _log_combine, rng)
            assert _rel(np.exp(np.logaddexp(LA + lh0, LH)), h[t]) < 1e-12


def test_log_reverse_operator_any_bracketing():
    # backward carry: w_s = a_s g_s with w_s = W + P w_{e+1} per chunk [s, e]
    rng = np.random.default_rng(10)
    inp = log_inputs(1, 37, 2, seed=10)
    la, lb, lh0, dh = (inp.log_a.astype(np.float64), inp.log_b.astype(np.float64),
                       inp.log_h0.astype(np.float64), inp.dh.astype(np.float64))
    dla, dlb, dlh0 = oracle.log_bwd(la, lb, lh0, dh)
    a = np.exp(la[0])
    b = np.exp(lb[0])
    g = dlb[0] / b                                   # g_t recovered from dlog b
    # element t: (P, W) = (a_t, a_t dh_t); combining (t) then (t+1 .. ) backwards
    def comb(x, y):  # x covers [s, m], y covers [m+1, e]:  w_s = Wx + Px (Wy + Py w)
        return x[0] * y[0], x[1] + x[0] * y[1]
    T = a.shape[0]
    for s in (0, 5, 36):
        for _ in range(5):
            P, W = _random_bracket_reduce([(a[u], a[u] * dh[0, u]) for u in range(s, T)], comb, rng)
            assert _rel(W, a[s] * g[s]) < 1e-12


def test_block_affine_operator_any_bracketing():
    rng = np.random.default_rng(12)
    inp = block_inputs(1, 24, 8, k=8, seed=12, h0="normal")
    A = inp.A[0, :, 0].astype(np.float64)
    b = inp.b[0].astype(np.float64)
    h0 = inp.h0[0].astype(np.float64)
    h = oracle.block_affine_fwd(inp.A, inp.b, inp.h0, 8)[0]
    def comb(x, y):  # x earlier, y later: (Phi_y Phi_x, Phi_y u_x + u_y)
        return y[0] @ x[0], y[0] @ x[1] + y[1]
    for t in (0, 9, 23):
        for _ in range(4):
            Phi, u = _random_bracket_reduce([(A[s], b[s]) for s in range(t + 1)], comb, rng)
            assert _rel(Phi @ h0 + u, h[t]) < 1e-12


# ------------------------------------------------ P6 norm preservation

def test_rotation_norm_and_orthogonality():
    inp = block_inputs(2, 200, 16, k=8, seed=13, gate=False, h0="normal")
    theta_free_A = inp.A.astype(np.float64)
    # rebuild the rotations exactly in fp64 from fresh angles so R is orthogonal to 1e-15
    rng = np.random.default_rng(13)
    theta = rng.uniform(-np.pi, np.pi, (2, 200, 2, 28))
    R = givens_mesh(theta, 8)
    h0 = inp.h0.astype(np.float64)
    h = oracle.block_affine_fwd(R, np.zeros((2, 200, 16)), h0, 8)
    n0 = np.linalg.norm(h0.reshape(2, 2, 8), axis=-1)
    nt = np.linalg.norm(h.reshape(2, 200, 2, 8), axis=-1)
    assert np.max(np.abs(nt - n0[:, None, :])) < 1e-12
    P = oracle.block_matrix_fwd(R, 8)
    PtP = np.einsum("btjrc,btjrd->btjcd", P, P)
    assert np.max(np.abs(PtP - np.eye(8))) < 1e-12
    assert theta_free_A.shape == R.shape


# -------------------------------------- P7 central finite differences, T <= 8

def _fd_check(f, grads, inputs, eps=1e-6, tol=1e-7):
    """f(*inputs) -> scalar loss; grads: list of analytic gradients per input."""
    for idx, (x, gx) in enumerate(zip(inputs, grads)):
        if x is None:
            continue
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


def test_log_gradients_finite_difference():
    inp = log_inputs(2, 6, 3, seed=14)
    la, lb, lh0, dh = (inp.log_a.astype(np.float64), inp.log_b.astype(np.float64),
                       inp.log_h0.astype(np.float64), inp.dh.astype(np.float64))
    loss = lambda la_, lb_, lh0_: float(np.sum(dh * oracle.log_fwd(la_, lb_, lh0_)))
    _fd_check(loss, oracle.log_bwd(la, lb, lh0, dh), [la, lb, lh0])


def test_block_affine_gradients_finite_difference():
    inp = block_inputs(2, 5, 8, k=4, seed=15, h0="normal")
    A, b, h0, dh = (inp.A.astype(np.float64), inp.b.astype(np.float64),
                    inp.h0.astype(np.float64), inp.dh.astype(np.float64))
    loss = lambda A_, b_, h0_: float(np.sum(dh * oracle.block_affine_fwd(A_, b_, h0_, 4)))
    _fd_check(loss, oracle.block_affine_bwd(A, b, h0, dh, 4), [A, b, h0])


def test_block_cumprod_gradients_finite_difference():
    inp = block_inputs(1, 6, 8, k=4, seed=16)
    A, dP = inp.A.astype(np.float64), inp.dP.astype(np.float64)
    loss = lambda A_: float(np.sum(dP * oracle.block_matrix_fwd(A_, 4)))
    _fd_check(loss, [oracle.block_matrix_bwd(A, dP, 4)], [A])


# --------------------------- P8 exact invariants at full configuration sizes

def test_log_invariants_full_size():
    for (B, T, d) in [(128, 64, 64), (16, 1024, 64)]:
        inp = log_inputs(B, T, d, seed=0)
        la, lb, lh0, dh = inp.log_a, inp.log_b, inp.log_h0, inp.dh.astype(np.float64)
        h = oracle.log_fwd(la, lb, lh0)
        dla, dlb, dlh0 = oracle.log_bwd(la, lb, lh0, dh)
        b = np.exp(lb.astype(np.float64))
        g = dlb / b
        # dlog a_t + dlog b_t = g_t h_t
        assert _rel(dla + dlb, g * h) < 1e-12
        # degree-1 homogeneity in (b, h0): sum dlog b + sum dlog h0 = sum dh * h
        lhs = dlb.sum() + dlh0.sum()
        rhs = float(np.sum(dh * h))
        assert abs(lhs - rhs) <= 1e-10 * np.sum(np.abs(dh * h))
        # g_T = dh_T and the reverse recurrence g_t = dh_t + a_{t+1} g_{t+1}
        a = np.exp(la.astype(np.float64))
        assert _rel(g[:, -1], dh[:, -1]) < 1e-13
        assert _rel(g[:, :-1], dh[:, :-1] + a[:, 1:] * g[:, 1:]) < 1e-12


def test_block_invariants_full_size():
    for (B, T) in [(128, 64), (16, 1024)]:
        inp = block_inputs(B, T, 64, k=8, seed=0, h0="normal")
        A, b, h0, dh, dP = inp.A, inp.b, inp.h0, inp.dh.astype(np.float64), inp.dP.astype(np.float64)
        h = oracle.block_affine_fwd(A, b, h0, 8)
        dA, db, dh0 = oracle.block_affine_bwd(A, b, h0, dh, 8)
        lhs = np.sum(db * b) + np.sum(dh0 * h0)
        rhs = np.sum(dh * h)
        assert abs(lhs - rhs) <= 1e-10 * np.sum(np.abs(dh * h))
        # dA_t = g_t h_{t-1}^T with g = db: rank-one structure
        hprev = np.concatenate([h0[:, None, :], h[:, :-1, :]], axis=1).reshape(B, T, 8, 8)
        assert _rel(dA, db.reshape(B, T, 8, 8)[..., :, None] * hprev[..., None, :]) < 1e-13
        P = oracle.block_matrix_fwd(A, 8)
        dAm = oracle.block_matrix_bwd(A, dP, 8)
        # P_t is homogeneous of degree t in A: sum <dA_t, A_t> = sum t <dP_t, P_t>
        t = np.arange(1, T + 1)[None, :, None]
        lhs = np.sum(dAm * A.astype(np.float64))
        rhs = np.sum(t * np.sum(dP * P, axis=(-1, -2)))
        assert abs(lhs - rhs) <= 1e-9 * np.sum(np.abs(t * np.sum(np.abs(dP * P), axis=(-1, -2))))


# ------------------------------ P9 directional derivative at full size (fp64)

def _directional(f, x_list, grads, v_list, eps):
    plus = [x + eps * v for x, v in zip(x_list, v_list)]
    minus = [x - eps * v for x, v in zip(x_list, v_list)]
    num = (f(*plus) - f(*minus)) / (2 * eps)
    ana = sum(float(np.sum(g * v)) for g, v in zip(grads, v_list))
    return num, ana


def test_log_directional_derivative_full_size():
    inp = log_inputs(128, 64, 64, seed=1)
    la, lb, lh0, dh = (x.astype(np.float64) for x in (inp.log_a, inp.log_b, inp.log_h0, inp.dh))
    rng = np.random.default_rng(100)
    v = [rng.standard_normal(x.shape) for x in (la, lb, lh0)]
    f = lambda a_, b_, c_: float(np.sum(dh * oracle.log_fwd(a_, b_, c_)))
    num, ana = _directional(f, [la, lb, lh0], oracle.log_bwd(la, lb, lh0, dh), v, 1e-5)
    assert abs(num - ana) <= 1e-7 * abs(ana)


def test_block_directional_derivative_full_size():
    inp = block_inputs(16, 1024, 64, k=8, seed=1, h0="normal")
    A, b, h0, dh, dP = (x.astype(np.float64) for x in (inp.A, inp.b, inp.h0, inp.dh, inp.dP))
    rng = np.random.default_rng(101)
    v = [rng.standard_normal(x.shape) * 0.01 for x in (A, b, h0)]
    f = lambda A_, b_, h0_: float(np.sum(dh * oracle.block_affine_fwd(A_, b_, h0_, 8)))
    num, ana = _directional(f, [A, b, h0], oracle.block_affine_bwd(A, b, h0, dh, 8), v, 1e-4)
    assert abs(num - ana) <= 1e-6 * abs(ana)
    vA = [rng.standard_normal(A.shape) * 0.01]
    fP = lambda A_: float(np.sum(dP * oracle.block_matrix_fwd(A_, 8)))
    num, ana = _directional(fP, [A], [oracle.block_matrix_bwd(A, dP, 8)], vA, 1e-4)
    assert abs(num - ana) <= 1e-6 * abs(ana)


# ----------------------------------------------- P10 sequence continuation

def test_sequence_continuation():
    inp = log_inputs(3, 50, 4, seed=17)
    h = oracle.log_fwd(inp.log_a, inp.log_b, inp.log_h0)
    h2 = oracle.log_fwd(inp.log_a[:, 20:], inp.log_b[:, 20:], np.log(h[:, 19]))
    assert _rel(h2, h[:, 20:]) < 1e-13
    binp = block_inputs(2, 40, 16, k=8, seed=18, h0="normal")
    hb = oracle.block_affine_fwd(binp.A, binp.b, binp.h0, 8)
    hb2 = oracle.block_affine_fwd(binp.A[:, 25:], binp.b[:, 25:], hb[:, 24], 8)
    assert _rel(hb2, hb[:, 25:]) < 1e-13
    P = oracle.block_matrix_fwd(binp.A, 8)
    P2 = oracle.block_matrix_fwd(binp.A[:, 25:], 8)
    assert _rel(np.einsum("btjrm,bjmc->btjrc", P2, P[:, 24]), P[:, 25:]) < 1e-12


def test_single_step():
    # T = 1: h_1 = a_1 h_0 + b_1 and every gradient is a single chain-rule term
    la = np.array([[[np.log(0.25)]]])
    lb = np.array([[[np.log(3.0)]]])
    lh0 = np.array([[np.log(2.0)]])
    h = oracle.log_fwd(la, lb, lh0)
    assert abs(h.ravel()[0] - 3.5) < 1e-14
    dla, dlb, dlh0 = oracle.log_bwd(la, lb, lh0, np.array([[[2.0]]]))
    assert abs(dla.ravel()[0] - 2 * 0.25 * 2.0) < 1e-15
    assert abs(dlb.ravel()[0] - 2 * 3.0) < 1e-14
    assert abs(dlh0.ravel()[0] - 2 * 0.25 * 2.0) < 1e-15
