"""Pins of the fp64 Givens angle-fused block-scan oracle (oracle.givens_fwd / givens_bwd).

Checked against: a hand-derived k = 2 example (tests/golden/givens_scan_worked.json);
the generator's own numpy mesh (synthetic.givens_mesh, code that shares nothing
with oracle.c) for the transition matrices; the separately pinned block-affine
oracle on those matrices for h, db and dh0; the chain rule with a numerical
derivative of the numpy mesh for dtheta and ds; and central finite differences
of the whole loss.
"""
import json
import os

import numpy as np

import oracle
from synthetic import block_inputs, givens_mesh

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rel(x, r):
    x, r = np.asarray(x, np.float64), np.asarray(r, np.float64)
    return float(np.max(np.abs(x - r)) / max(np.max(np.abs(r)), 1e-300))


def _sig(u):
    return 1.0 / (1.0 + np.exp(-u))


def _inputs(B, T, d, k, seed):
    inp = block_inputs(B, T, d, k=k, seed=seed, h0="normal", return_angles=True)
    return (inp.theta.astype(np.float64), inp.s.astype(np.float64), inp.b.astype(np.float64),
            inp.h0.astype(np.float64), inp.dh.astype(np.float64))


def test_golden_k2():
    fx = json.load(open(os.path.join(GOLD, "givens_scan_worked.json")))
    th = np.array(fx["theta"]).reshape(1, 1, 1, 1)
    s = np.array([[[fx["s"]]]])
    b = np.array(fx["b"]).reshape(1, 1, 2)
    h0 = np.array(fx["h0"]).reshape(1, 2)
    dh = np.array(fx["dh"]).reshape(1, 1, 2)
    np.testing.assert_allclose(oracle.givens_fwd(th, s, b, h0, 2).ravel(), fx["h"], rtol=0, atol=1e-15)
    dth, ds, db, dh0 = oracle.givens_bwd(th, s, b, h0, dh, 2)
    np.testing.assert_allclose(dth.ravel(), fx["dtheta"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(ds.ravel(), [fx["ds"]], rtol=0, atol=1e-15)
    np.testing.assert_allclose(db.ravel(), fx["db"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(dh0.ravel(), fx["dh0"], rtol=0, atol=1e-15)


def test_matrices_match_numpy_mesh():
    th, s, _, _, _ = _inputs(2, 5, 16, 8, 51)
    A = oracle.givens_matrix(th, s, 8)
    assert _rel(A, _sig(s)[..., None, None] * givens_mesh(th, 8)) < 1e-14


def test_forward_and_vector_gradients_match_block_affine_oracle():
    th, s, b, h0, dh = _inputs(3, 40, 16, 8, 52)
    A = _sig(s)[..., None, None] * givens_mesh(th, 8)
    assert _rel(oracle.givens_fwd(th, s, b, h0, 8), oracle.block_affine_fwd(A, b, h0, 8)) < 1e-13
    _, _, db, dh0 = oracle.givens_bwd(th, s, b, h0, dh, 8)
    _, rdb, rdh0 = oracle.block_affine_bwd(A, b, h0, dh, 8)
    assert _rel(db, rdb) < 1e-13 and _rel(dh0, rdh0) < 1e-13


def test_angle_and_gate_gradients_by_chain_rule():
    """dtheta = sigmoid(s) <dA, dR/dtheta> with dR/dtheta by central differences of the numpy mesh;
    ds = sigmoid'(s) <dA, R>; dA from the block-affine oracle."""
    th, s, b, h0, dh = _inputs(2, 6, 16, 8, 53)
    R = givens_mesh(th, 8)
    A = _sig(s)[..., None, None] * R
    dA, _, _ = oracle.block_affine_bwd(A, b, h0, dh, 8)
    dth, ds, _, _ = oracle.givens_bwd(th, s, b, h0, dh, 8)
    assert _rel(ds, _sig(s) * (1 - _sig(s)) * np.sum(dA * R, axis=(-1, -2))) < 1e-12
    eps = 1e-6
    ref = np.empty_like(th)
    for a in range(th.shape[-1]):
        tp, tm = th.copy(), th.copy()
        tp[..., a] += eps
        tm[..., a] -= eps
        dR = (givens_mesh(tp, 8) - givens_mesh(tm, 8)) / (2 * eps)
        ref[..., a] = _sig(s) * np.sum(dA * dR, axis=(-1, -2))
    assert np.max(np.abs(dth - ref)) / max(1.0, np.max(np.abs(ref))) < 1e-8


def test_gradients_finite_difference():
    th, s, b, h0, dh = _inputs(1, 4, 8, 4, 54)
    loss = lambda th_, s_, b_, h0_: float(np.sum(dh * oracle.givens_fwd(th_, s_, b_, h0_, 4)))
    grads = oracle.givens_bwd(th, s, b, h0, dh, 4)
    eps = 1e-6
    for v, gv in zip((th, s, b, h0), grads):
        flat = v.reshape(-1)
        num = np.empty_like(flat)
        for i in range(flat.size):
            old = flat[i]
            flat[i] = old + eps
            fp = loss(th, s, b, h0)
            flat[i] = old - eps
            fm = loss(th, s, b, h0)
            flat[i] = old
            num[i] = (fp - fm) / (2 * eps)
        assert np.max(np.abs(num - gv.reshape(-1))) / max(1.0, np.max(np.abs(gv))) < 1e-7


def test_rotation_only_preserves_norm():
    """s -> +inf (gate 1) and b = 0: ||h_t|| = ||h0|| for every t."""
    th, _, b, h0, _ = _inputs(2, 30, 16, 8, 55)
    s = np.full(th.shape[:3], 60.0)
    h = oracle.givens_fwd(th, s, np.zeros_like(b), h0, 8)
    n0 = np.linalg.norm(h0.reshape(2, 2, 8), axis=-1)
    nt = np.linalg.norm(h.reshape(2, 30, 2, 8), axis=-1)
    assert np.max(np.abs(nt - n0[:, None])) < 1e-12
