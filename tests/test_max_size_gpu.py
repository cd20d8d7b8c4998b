"""Tensors at the boundary's size limit (2^31 - 1 elements per tensor).

The largest tensor of each op sits just under the limit, with ragged shapes
(a d that is not a multiple of the 64 chains a log-space workgroup row holds,
a T that leaves the last block tile 127 steps long).  The inputs are drawn on
the GPU (synthetic.device_*_inputs, seeded).  Two checks:
  * every element of every output is written with a finite value: outputs are
    filled with NaN before the call, so an element that no lane stores (or a
    store that lands in the wrong place) is caught anywhere in the tensor;
  * sampled chains -- the first and last ones (whose element offsets reach the
    top of the 31-bit range), chains on either side of a workgroup boundary and
    random ones -- match the fp64 oracle run on that chain alone, under the
    floored relative-error rule of the parity tests.
Two shapes per op where the carry matters: a wide one (many chains, a few
tiles along T) and the longest sequence at the limit (16384 log-space or
32768 block tiles along T, so each carry crosses every tile of the sequence
through the look-back).  The same kernels and launch shapes run as at the
benchmark's sizes; only the grids are larger (up to 262144 workgroups).
"""
import gc

import numpy as np
import pytest

import oracle
from synthetic import device_block_inputs, device_log_inputs
from tests.test_parity_gpu import BLOCK_TOL, LOG_TOL, floored_err, say, ws_clean

pytestmark = pytest.mark.gpu

LIMIT = 2 ** 31 - 1
LOG_SHAPE = (2, 1024, 1048575)    # 2,147,481,600 elements per (B,T,d) tensor
BLOCK_SHAPE = (8208, 511, 64, 8)  # A: 2,147,475,456 elements; T = 3 * 128 + 127
# the longest sequences at the limit: 16384 (log) and 32768 (block) tiles along T
LOG_LONG = (1, 1 << 21, 1023)          # 2,145,386,496 elements
BLOCK_LONG = (1, (1 << 22) - 1, 64, 8)  # A: 2,147,483,136 elements


def _free():
    import torch
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _nan_like(t):
    import torch
    return torch.full_like(t, float("nan"))


def _all_finite(name, t):
    import torch
    assert bool(torch.isfinite(t).all()), f"{name}: an element is unwritten or not finite"


def _sample(n_hi, fixed, count, seed):
    rng = np.random.default_rng(seed)
    extra = [int(x) for x in rng.integers(0, n_hi, count)]
    return list(dict.fromkeys(fixed + extra))


@pytest.mark.parametrize("shape", [LOG_SHAPE, LOG_LONG], ids=["wide", "longT"])
def test_log_scan_at_size_limit(gpu, shape):
    import scan_linear_rnns_amd as mgs
    B, T, d = shape
    assert LIMIT - (1 << 22) < B * T * d <= LIMIT
    say(f"log scan at the size limit B={B} T={T} d={d}")
    try:
        la, lb, lh0, dh = device_log_inputs(B, T, d, gpu, seed=5)
        h, ws = mgs.mgs_scan_log_fwd(la, lb, lh0, h=_nan_like(la))
        out = (_nan_like(la), _nan_like(la), _nan_like(lh0))
        dla, dlb, dlh0 = mgs.mgs_scan_log_bwd(la, lb, lh0, dh, ws=ws, fwd_state_valid=True, out=out)
        ws_clean(ws)
        for name, t in (("h", h), ("dlog_a", dla), ("dlog_b", dlb), ("dlog_h0", dlh0)):
            _all_finite(name, t)
        fixed = [0, 1, 63, 64, d - 1, d, d + 63, 2 * d - 65, 2 * d - 2, 2 * d - 1]
        flat = _sample(B * d, [c for c in fixed if c < B * d], 8 if T <= 4096 else 2, 5)
        for ch in flat:
            bb, c = divmod(ch, d)
            col = lambda t: t[bb, :, c].cpu().numpy()[None, :, None]
            a_c, b_c, g_c = col(la), col(lb), col(dh)
            h0_c = lh0[bb, c].reshape(1, 1).cpu().numpy()
            rh = oracle.log_fwd(a_c, b_c, h0_c)
            rda, rdb, rdh0 = oracle.log_bwd(a_c, b_c, h0_c, g_c)
            got = dict(h=col(h), dlog_a=col(dla), dlog_b=col(dlb), dlog_h0=dlh0[bb, c].reshape(1, 1).cpu().numpy())
            ref = dict(h=rh, dlog_a=rda, dlog_b=rdb, dlog_h0=rdh0)
            for key in got:
                e = floored_err(got[key], ref[key])
                assert e <= LOG_TOL, (ch, key, e)
    finally:
        la = lb = lh0 = dh = h = ws = out = dla = dlb = dlh0 = None
        _free()


def _block_chain(t, bb, jb, k):
    """(1, T, 1, k, k) slice of an A-shaped tensor or (1, T, k) of a vector one."""
    if t.dim() == 5:
        return t[bb, :, jb].cpu().numpy()[None, :, None]
    return t[bb, :, jb * k:(jb + 1) * k].cpu().numpy()[None]


def _block_chains(B, T, nb):
    fixed = [x for x in (0, 1, 3, 4, 7, B * nb - 5, B * nb - 4, B * nb - 1) if 0 <= x < B * nb]
    if T > 4096:
        fixed = [0, B * nb - 1]
    return [divmod(x, nb) for x in _sample(B * nb, fixed, 8 if T <= 4096 else 0, 6)]


@pytest.mark.parametrize("shape", [BLOCK_SHAPE, BLOCK_LONG], ids=["wide", "longT"])
def test_block_affine_at_size_limit(gpu, shape):
    import torch
    import scan_linear_rnns_amd as mgs
    B, T, d, k = shape
    nb = d // k
    assert LIMIT - 65536 < B * T * d * k <= LIMIT
    say(f"block-affine scan at the size limit B={B} T={T} d={d} k={k}")
    try:
        x = device_block_inputs(B, T, d, k, gpu, seed=6)
        A, b, dh = x["A"], x["b"], x["dh"]
        h, ws = mgs.mgs_block_affine_scan_fwd(A, b, None, k=k, h=_nan_like(b))
        out = (_nan_like(A), _nan_like(b), torch.full((B, d), float("nan"), device=gpu))
        dA, db, dh0 = mgs.mgs_block_affine_scan_bwd(A, b, None, h, dh, k=k, ws=ws, out=out)
        ws_clean(ws)
        for name, t in (("h", h), ("dA", dA), ("db", db), ("dh0", dh0)):
            _all_finite(name, t)
        for bb, jb in _block_chains(B, T, nb):
            A_c, b_c, g_c = (_block_chain(t, bb, jb, k) for t in (A, b, dh))
            rh = oracle.block_affine_fwd(A_c, b_c, None, k)
            rdA, rdb, rdh0 = oracle.block_affine_bwd(A_c, b_c, None, g_c, k)
            got = dict(h=_block_chain(h, bb, jb, k), dA=_block_chain(dA, bb, jb, k), db=_block_chain(db, bb, jb, k),
                       dh0=dh0[bb, jb * k:(jb + 1) * k].cpu().numpy()[None])
            ref = dict(h=rh, dA=rdA, db=rdb, dh0=rdh0)
            for key in got:
                e = floored_err(got[key], ref[key])
                assert e <= BLOCK_TOL, ((bb, jb), key, e)
    finally:
        x = A = b = dh = h = ws = out = dA = db = dh0 = None
        _free()


def test_block_cumprod_at_size_limit(gpu):
    import scan_linear_rnns_amd as mgs
    B, T, d, k = BLOCK_SHAPE
    nb = d // k
    say(f"block cumulative product at the size limit B={B} T={T} d={d} k={k}")
    try:
        x = device_block_inputs(B, T, d, k, gpu, seed=7, with_b=False, with_dh=False, with_dP=True)
        A, dP = x["A"], x["dP"]
        P, ws = mgs.mgs_block_matrix_scan_fwd(A, k=k, P=_nan_like(A))
        dA = mgs.mgs_block_matrix_scan_bwd(A, dP, k=k, ws=ws, fwd_state_valid=True, dA=_nan_like(A))
        ws_clean(ws)
        _all_finite("P", P)
        _all_finite("dA", dA)
        for bb, jb in _block_chains(B, T, nb):
            A_c, g_c = _block_chain(A, bb, jb, k), _block_chain(dP, bb, jb, k)
            rP = oracle.block_matrix_fwd(A_c, k)
            rdA = oracle.block_matrix_bwd(A_c, g_c, k)
            for key, got, ref in (("P", _block_chain(P, bb, jb, k), rP), ("dA", _block_chain(dA, bb, jb, k), rdA)):
                e = floored_err(got, ref)
                assert e <= BLOCK_TOL, ((bb, jb), key, e)
    finally:
        x = A = dP = P = ws = dA = None
        _free()
