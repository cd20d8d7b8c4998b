"""GPU parity of the block scans at every block size of the envelope other than
k = 8 (k = 1, 2, 4, 16; k = 8 is covered by tests/test_parity_gpu.py).

Same rule and bar as the k = 8 block tests: every output tensor element by
element against the fp64 oracle on the same fp32 inputs,
err = max_i |x_i - r_i| / max(|r_i|, 1e-3 * max_j |r_j|) <= 2e-4.  Inputs:
the gated Givens-mesh generator at block size k (A = sigmoid(s) R(theta) with
k(k-1)/2 angles per block; for k = 1, A = sigmoid(s)).
"""
import numpy as np
import pytest

import oracle
from synthetic import block_inputs, log_inputs
from tests.test_parity_gpu import BLOCK_TOL, floored_err, say, to_dev, to_np, ws_clean

pytestmark = pytest.mark.gpu

KS = [1, 2, 4, 16]


def run_block_k(B, T, d, k, seed, dev, *, gate=True, h0="zero", matrix=True):
    import scan_linear_rnns_amd as mgs
    inp = block_inputs(B, T, d, k=k, seed=seed, gate=gate, h0=h0, with_dP=matrix)
    A, b, h0t, dh = (to_dev(x, dev) for x in (inp.A, inp.b, inp.h0, inp.dh))
    h, ws = mgs.mgs_block_affine_scan_fwd(A, b, h0t, k=k)
    dA, db, dh0 = mgs.mgs_block_affine_scan_bwd(A, b, h0t, h, dh, k=k, ws=ws)
    ws_clean(ws)
    out = dict(h=to_np(h), dA=to_np(dA), db=to_np(db), dh0=to_np(dh0))
    ref = dict(h=oracle.block_affine_fwd(inp.A, inp.b, inp.h0, k))
    ref["dA"], ref["db"], ref["dh0"] = oracle.block_affine_bwd(inp.A, inp.b, inp.h0, inp.dh, k)
    if matrix:
        dP = to_dev(inp.dP, dev)
        P, wsm = mgs.mgs_block_matrix_scan_fwd(A, k=k)
        dAm = mgs.mgs_block_matrix_scan_bwd(A, dP, k=k, ws=wsm, fwd_state_valid=True)
        ws_clean(wsm)
        out["P"], out["dA_matrix"] = to_np(P), to_np(dAm)
        ref["P"] = oracle.block_matrix_fwd(inp.A, k)
        ref["dA_matrix"] = oracle.block_matrix_bwd(inp.A, inp.dP, k)
    return out, ref


def check(out, ref, tol=BLOCK_TOL):
    for key in out:
        e = floored_err(out[key], ref[key])
        assert e <= tol, (key, e)


SHAPES = [("lab", 128, 64, 64), ("longT", 16, 1024, 64)]


@pytest.mark.parametrize("k", KS)
@pytest.mark.parametrize("name,B,T,d", SHAPES, ids=[s[0] for s in SHAPES])
def test_blocksize_configs(gpu, name, B, T, d, k):
    say(f"block k={k} {name} B={B} T={T} d={d}")
    out, ref = run_block_k(B, T, d, k, 0, gpu)
    check(out, ref)


# d ragged against the 32/k chains a half-wave holds, T ragged against the tiles
EDGES = [(1, 1, 1, 1), (3, 7, 3, 1), (2, 300, 37, 1), (1, 2048, 5, 1),
         (1, 1, 2, 2), (3, 65, 6, 2), (2, 129, 34, 2),
         (1, 2, 4, 4), (3, 63, 12, 4), (2, 300, 20, 4), (1, 1000, 4, 4),
         (1, 1, 16, 16), (3, 7, 16, 16), (2, 12, 32, 16), (2, 65, 48, 16), (1, 200, 16, 16), (1, 300, 32, 16),
         (1, 1000, 16, 16)]


@pytest.mark.parametrize("B,T,d,k", EDGES)
def test_blocksize_edges(gpu, B, T, d, k):
    say(f"block k={k} edge B={B} T={T} d={d}")
    out, ref = run_block_k(B, T, d, k, 6, gpu, h0="normal")
    check(out, ref)


# k = 16: the forward and the backward tile T differently (forward chunks of up
# to 8 steps, backward chunks of up to 4; T = 12 gives a backward chunk longer
# than the forward's, T = 200 a two-tile forward saving states inside its chunks)
@pytest.mark.parametrize("k,B,T,d", [(1, 2, 7, 3), (2, 4, 1024, 64), (4, 3, 300, 12), (16, 2, 1024, 32),
                                     (16, 2, 12, 32), (16, 1, 200, 16)])
def test_blocksize_matrix_bwd_without_forward_state(gpu, k, B, T, d):
    """A fresh workspace: the backward recomputes the chunk states itself and
    gives the oracle's dA, bit for bit the same as with the forward's states."""
    import torch
    import scan_linear_rnns_amd as mgs
    say(f"matrix bwd recompute-states k={k} B={B} T={T} d={d}")
    inp = block_inputs(B, T, d, k=k, seed=17)
    A, dP = to_dev(inp.A, gpu), to_dev(inp.dP, gpu)
    dA_fresh = mgs.mgs_block_matrix_scan_bwd(A, dP, k=k)
    P, wsm = mgs.mgs_block_matrix_scan_fwd(A, k=k)
    dA_reuse = mgs.mgs_block_matrix_scan_bwd(A, dP, k=k, ws=wsm, fwd_state_valid=True)
    ws_clean(wsm)
    assert floored_err(to_np(dA_fresh), oracle.block_matrix_bwd(inp.A, inp.dP, k)) <= BLOCK_TOL
    assert torch.equal(dA_fresh, dA_reuse)


@pytest.mark.parametrize("k,T", [(2, 1024), (4, 1024), (16, 1024), (4, 2000)])
def test_blocksize_rotation_only_long_T(gpu, k, T):
    """Pure rotations (no gate): P stays orthogonal over T steps.  Held to the
    normwise bar of the k = 8 rotation-only test (entries near zero carry the
    rounding of O(1) partial results, see there).  k = 16 at T = 1024 and
    k = 4 at T = 2000 have more tiles along T than waves per workgroup, so the
    look-back also composes far tiles."""
    say(f"block k={k} rotation-only T={T}")
    out, ref = run_block_k(2, T, 32, k, 9, gpu, gate=False, h0="normal")
    for key in out:
        x, r = out[key].astype(np.float64), ref[key]
        assert np.all(np.isfinite(x))
        assert np.max(np.abs(x - r)) / np.max(np.abs(r)) <= 2e-5, key
    P = out["P"].astype(np.float64)
    PtP = np.einsum("btjrc,btjrd->btjcd", P, P)
    assert np.max(np.abs(PtP - np.eye(k))) < 1e-4


@pytest.mark.parametrize("B,T,d", [(128, 64, 64), (16, 1024, 64), (3, 300, 5)])
def test_k1_block_affine_matches_log_scan(gpu, B, T, d):
    """k = 1 block-affine with A > 0 is the log-space scan with log a = log A:
    the two GPU ops agree on h, and their gradients satisfy the chain rule
    dlog a = A dA, dlog b = b db, dlog h0 = h0 dh0 (a cross-op check of two
    independent kernels)."""
    import torch
    import scan_linear_rnns_amd as mgs
    say(f"k=1 block-affine vs log scan B={B} T={T} d={d}")
    inp = log_inputs(B, T, d, seed=21)
    la, lb, lh0, dh = (to_dev(x, gpu) for x in (inp.log_a, inp.log_b, inp.log_h0, inp.dh))
    h_log, ws = mgs.mgs_scan_log_fwd(la, lb, lh0)
    dla, dlb, dlh0 = mgs.mgs_scan_log_bwd(la, lb, lh0, dh, ws=ws, fwd_state_valid=True)
    ws_clean(ws)
    A = torch.exp(la).reshape(B, T, d, 1, 1).contiguous()
    b = torch.exp(lb).contiguous()
    h0 = torch.exp(lh0).contiguous()
    h_blk, wsb = mgs.mgs_block_affine_scan_fwd(A, b, h0, k=1)
    dA, db, dh0 = mgs.mgs_block_affine_scan_bwd(A, b, h0, h_blk, dh, k=1, ws=wsb)
    ws_clean(wsb)
    assert floored_err(to_np(h_blk), to_np(h_log)) <= 1e-4
    assert floored_err(to_np(dA.reshape(B, T, d) * A.reshape(B, T, d)), to_np(dla)) <= 1e-4
    assert floored_err(to_np(db * b), to_np(dlb)) <= 1e-4
    assert floored_err(to_np(dh0 * h0), to_np(dlh0)) <= 1e-4
