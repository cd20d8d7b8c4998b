"""Pins of the delta-rule oracle (oracle.delta_fwd), independent of the oracle's loop.

The delta rule of DeltaMinGRU (minGRU home page: DeltaMinGRU reimplements
DeltaNet, Yang et al. 2024, and runs its chunked WY form as the parallel
forward): S_t = S_{t-1} + beta_t (v_t - S_{t-1} k_t) k_t^T, o_t = S_t q_t.

  * a worked example derived by hand (tests/golden/delta_rule_worked.json);
  * the closed form S_t = S_0 H_1 .. H_t + sum_s beta_s v_s k_s^T H_{s+1} .. H_t
    with H_s = I - beta_s k_s k_s^T, built from numpy matrix products;
  * special cases: beta = 0 keeps the state; beta = 1 with a unit key writes
    v exactly (S k = v); orthonormal keys with beta = 1 make the state a table
    of the last value written under each key;
  * linearity of (o, S_T) in (v, S_0); sequence continuation;
  * the chunked WY re-association (the form the GPU kernels evaluate), in
    numpy, agrees with the loop.
"""
import json
import os

import numpy as np
import pytest

import oracle
from synthetic import delta_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "delta_rule_worked.json")


def test_golden_delta_rule():
    g = json.load(open(GOLDEN))
    o, ST = oracle.delta_fwd(np.array(g["q"]), np.array(g["k"]), np.array(g["v"]), np.array(g["beta"]))
    np.testing.assert_allclose(o, np.array(g["o"]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(ST, np.array(g["ST"]), rtol=0, atol=1e-14)


def _closed_form_states(q, k, v, beta, S0):
    """S_1..S_T from products of the H_s, one prefix at a time."""
    B, T, dk = k.shape
    dv = v.shape[2]
    out = np.zeros((B, T, dv, dk))
    for b in range(B):
        H = [np.eye(dk) - beta[b, s] * np.outer(k[b, s], k[b, s]) for s in range(T)]
        for t in range(T):
            St = S0[b].copy()
            for s in range(t + 1):
                St = St @ H[s]
            for s in range(t + 1):
                term = beta[b, s] * np.outer(v[b, s], k[b, s])
                for r in range(s + 1, t + 1):
                    term = term @ H[r]
                St = St + term
            out[b, t] = St
    return out


def test_closed_form_householder_products():
    rng = np.random.default_rng(3)
    B, T, dk, dv = 2, 6, 3, 4
    q = rng.standard_normal((B, T, dk))
    k = rng.standard_normal((B, T, dk))          # not normalised: the identity holds for any k
    v = rng.standard_normal((B, T, dv))
    beta = rng.uniform(0.1, 1.5, (B, T))
    S0 = rng.standard_normal((B, dv, dk))
    o, ST = oracle.delta_fwd(q, k, v, beta, S0)
    S = _closed_form_states(q, k, v, beta, S0)
    np.testing.assert_allclose(ST, S[:, -1], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(o, np.einsum("btrc,btc->btr", S, q), rtol=1e-12, atol=1e-12)


def test_beta_zero_keeps_state():
    inp = delta_inputs(2, 9, 5, seed=4, s0="normal")
    beta = np.zeros_like(inp.beta)
    o, ST = oracle.delta_fwd(inp.q, inp.k, inp.v, beta, inp.S0)
    S0 = inp.S0.astype(np.float64)
    np.testing.assert_allclose(ST, S0, rtol=0, atol=0)
    np.testing.assert_allclose(o, np.einsum("brc,btc->btr", S0, inp.q.astype(np.float64)), rtol=1e-13, atol=1e-13)


def test_unit_key_full_write():
    """beta = 1 and |k| = 1 make I - k k^T a projection: S_1 k_1 = v_1 whatever S_0."""
    inp = delta_inputs(3, 1, 6, seed=5, s0="normal")
    k = inp.k.astype(np.float64)
    k = k / np.linalg.norm(k, axis=-1, keepdims=True)
    _, ST = oracle.delta_fwd(inp.q, k, inp.v, np.ones((3, 1)), inp.S0)
    np.testing.assert_allclose(np.einsum("brc,bc->br", ST, k[:, 0]), inp.v[:, 0], rtol=1e-12, atol=1e-12)


def test_orthonormal_keys_are_a_table():
    """Keys e_{perm(t)} with beta = 1: column j of S_T is the last value written
    under key j, or S_0's column j if none was."""
    rng = np.random.default_rng(6)
    B, T, dk, dv = 2, 11, 4, 3
    keys = rng.integers(0, dk - 1, (B, T))        # key dk-1 is never written
    k = np.zeros((B, T, dk))
    for b in range(B):
        k[b, np.arange(T), keys[b]] = 1.0
    v = rng.standard_normal((B, T, dv))
    q = rng.standard_normal((B, T, dk))
    S0 = rng.standard_normal((B, dv, dk))
    _, ST = oracle.delta_fwd(q, k, v, np.ones((B, T)), S0)
    for b in range(B):
        for j in range(dk):
            ts = np.nonzero(keys[b] == j)[0]
            want = S0[b][:, j] if len(ts) == 0 else v[b, ts[-1]]
            np.testing.assert_allclose(ST[b][:, j], want, rtol=0, atol=1e-15)


def test_linearity_in_values_and_state():
    i1 = delta_inputs(2, 7, 5, seed=7, s0="normal")
    i2 = delta_inputs(2, 7, 5, seed=8, s0="normal")
    a = -1.75
    v = a * i1.v.astype(np.float64) + i2.v
    S0 = a * i1.S0.astype(np.float64) + i2.S0
    o, ST = oracle.delta_fwd(i1.q, i1.k, v, i1.beta, S0)
    o1, S1 = oracle.delta_fwd(i1.q, i1.k, i1.v, i1.beta, i1.S0)
    o2, S2 = oracle.delta_fwd(i1.q, i1.k, i2.v, i1.beta, i2.S0)
    np.testing.assert_allclose(o, a * o1 + o2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(ST, a * S1 + S2, rtol=1e-12, atol=1e-12)


def test_sequence_continuation():
    inp = delta_inputs(2, 30, 8, seed=9, s0="normal")
    o, ST = oracle.delta_fwd(inp.q, inp.k, inp.v, inp.beta, inp.S0)
    oa, Sa = oracle.delta_fwd(inp.q[:, :13], inp.k[:, :13], inp.v[:, :13], inp.beta[:, :13], inp.S0)
    ob, Sb = oracle.delta_fwd(inp.q[:, 13:], inp.k[:, 13:], inp.v[:, 13:], inp.beta[:, 13:], Sa)
    np.testing.assert_allclose(np.concatenate([oa, ob], axis=1), o, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(Sb, ST, rtol=1e-13, atol=1e-13)


def _chunked_wy(q, k, v, beta, S0, C):
    """The chunked WY re-association, per chunk of C steps from the entering state S:
    G = K K^T; U', W solve (I + strict_lower(diag(beta) G)) [U' W] = diag(beta) [V K];
    then the state-dependent pieces: X = U' - W S^T, O = Q S^T + causal(Q K^T) X,
    S <- S + X^T K."""
    q, k, v, beta = (np.asarray(x, np.float64) for x in (q, k, v, beta))
    B, T, dk = k.shape
    dv = v.shape[2]
    o = np.zeros((B, T, dv))
    ST = np.zeros((B, dv, dk))
    for b in range(B):
        S = np.zeros((dv, dk)) if S0 is None else np.asarray(S0[b], np.float64).copy()
        for s in range(0, T, C):
            Q, K, V, be = q[b, s:s + C], k[b, s:s + C], v[b, s:s + C], beta[b, s:s + C]
            n = K.shape[0]
            L = np.eye(n) + np.tril(be[:, None] * (K @ K.T), -1)
            U = np.linalg.solve(L, be[:, None] * V)
            W = np.linalg.solve(L, be[:, None] * K)
            X = U - W @ S.T
            o[b, s:s + C] = Q @ S.T + np.tril(Q @ K.T) @ X
            S = S + X.T @ K
        ST[b] = S
    return o, ST


@pytest.mark.parametrize("C", [1, 4, 16])
def test_chunked_wy_matches_loop(C):
    inp = delta_inputs(2, 37, 16, seed=10, s0="normal")
    o, ST = oracle.delta_fwd(inp.q, inp.k, inp.v, inp.beta, inp.S0)
    ow, Sw = _chunked_wy(inp.q, inp.k, inp.v, inp.beta, inp.S0, C)
    np.testing.assert_allclose(ow, o, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(Sw, ST, rtol=1e-11, atol=1e-11)
