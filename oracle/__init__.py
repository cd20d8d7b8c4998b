"""fp64 CPU oracle for the minGRU scan engine -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never calls it, and
it shares no code with the GPU path: the arithmetic lives in ``oracle.c``
(plain sequential loops over t in double precision), compiled with gcc into
``liboracle.so`` next to this file.  This module only widens the fp32 inputs to
float64 (exactly), calls the C loops and returns float64 results.

What each function follows is stated in ``oracle.c``:
  * ``log_fwd`` / ``log_bwd`` -- the minGRU linear recurrence
    h_t = a_t h_{t-1} + b_t with inputs log a_t, log b_t, log h_0
    (minGRU home page, introduction: the log-space baseline MinGRU and its
    Heinsen scan); gradients by the chain rule.
  * ``linear_fwd`` / ``linear_bwd`` -- the same recurrence in linear space,
    a_t of either sign (linear_scan in the home page's speed-up table and in
    the how-to's Step 2 table; SignedMinGRU's signed gates on the home page).
  * ``mingru_fwd`` / ``mingru_bwd`` -- the minGRU cell ahead of the scan
    (a = sigmoid(-k), b = (1 - a) g(x), h_0 = g(x0); home page, introduction)
    followed by the same recurrence; gradients for k, x, x0.
  * ``givens_fwd`` / ``givens_bwd`` -- the block-affine scan with
    A_t = sigmoid(s_t) R(theta_t) formed from angles and gate (GivensMinGRU on
    the home page; the fused backward of the how-to's Step 3); gradients for
    theta, s, b, h0.
  * ``block_affine_fwd`` / ``block_affine_bwd`` -- h_t = A_t h_{t-1} + b_t
    with block-diagonal k x k transitions (matrix_affine_scan in the
    "Run the benchmarks" how-to, Step 2; RotationMinGRU / GivensMinGRU on the
    home page).
  * ``block_matrix_fwd`` / ``block_matrix_bwd`` -- P_t = A_t P_{t-1},
    P_0 = I (matrix_scan in the same table).
  * ``delta_fwd`` -- the delta rule of DeltaMinGRU (home page: DeltaNet's
    recurrence, whose chunked WY form is the parallel forward):
    S_t = S_{t-1} + beta_t (v_t - S_{t-1} k_t) k_t^T, o_t = S_t q_t.

Parity pins: every function here is pinned against closed forms, special
cases reducing to numpy routines, brute-force products, finite differences and
exact invariants in ``tests/test_oracle_pins.py`` and the hand-derived
fixtures under ``tests/golden/``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
# MGS_ORACLE_LIBRARY: an already built copy of oracle.c to load instead (the
# sanitizer test loads one built with address and undefined-behaviour checks)
_LIB = os.environ.get("MGS_ORACLE_LIBRARY", os.path.join(_HERE, "liboracle.so"))
_lock = threading.Lock()
_lib = None

_D = ctypes.POINTER(ctypes.c_double)
_I = ctypes.c_int64


def build(force: bool = False) -> str:
    """Compile oracle.c with gcc (no fast-math; IEEE double arithmetic)."""
    if "MGS_ORACLE_LIBRARY" in os.environ:
        return _LIB
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-std=c99",
               "-shared", "-fPIC", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            lib = ctypes.CDLL(_LIB)
            sig = {
                "oracle_log_fwd": [_D, _D, _D, _D, _I, _I, _I],
                "oracle_log_bwd": [_D, _D, _D, _D, _D, _D, _D, _I, _I, _I],
                "oracle_linear_fwd": [_D, _D, _D, _D, _I, _I, _I],
                "oracle_linear_bwd": [_D, _D, _D, _D, _D, _D, _D, _I, _I, _I],
                "oracle_mingru_fwd": [_D, _D, _D, _D, _I, _I, _I],
                "oracle_mingru_bwd": [_D, _D, _D, _D, _D, _D, _D, _I, _I, _I],
                "oracle_givens_fwd": [_D, _D, _D, _D, _D, _I, _I, _I, _I],
                "oracle_givens_bwd": [_D, _D, _D, _D, _D, _D, _D, _D, _D, _I, _I, _I, _I],
                "oracle_block_affine_fwd": [_D, _D, _D, _D, _I, _I, _I, _I],
                "oracle_block_affine_bwd": [_D, _D, _D, _D, _D, _D, _D, _I, _I, _I, _I],
                "oracle_block_matrix_fwd": [_D, _D, _I, _I, _I, _I],
                "oracle_block_matrix_bwd": [_D, _D, _D, _I, _I, _I, _I],
                "oracle_delta_fwd": [_D, _D, _D, _D, _D, _D, _D, _I, _I, _I, _I],
            }
            for name, args in sig.items():
                fn = getattr(lib, name)
                fn.argtypes = args
                fn.restype = None
            _lib = lib
    return _lib


def _f64(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _p(x):
    return None if x is None else x.ctypes.data_as(_D)


def log_fwd(log_a, log_b, log_h0):
    """h (B,T,d) of the log-space scan; inputs (B,T,d), (B,T,d), (B,d)."""
    la, lb, lh0 = _f64(log_a), _f64(log_b), _f64(log_h0)
    B, T, d = la.shape
    assert lb.shape == la.shape and lh0.shape == (B, d)
    h = np.empty((B, T, d), np.float64)
    _load().oracle_log_fwd(_p(la), _p(lb), _p(lh0), _p(h), B, T, d)
    return h


def log_bwd(log_a, log_b, log_h0, dh):
    """(dlog_a, dlog_b, dlog_h0) for L = sum(dh * h)."""
    la, lb, lh0, g = _f64(log_a), _f64(log_b), _f64(log_h0), _f64(dh)
    B, T, d = la.shape
    assert lb.shape == la.shape and g.shape == la.shape and lh0.shape == (B, d)
    dla = np.empty_like(la)
    dlb = np.empty_like(la)
    dlh0 = np.empty_like(lh0)
    _load().oracle_log_bwd(_p(la), _p(lb), _p(lh0), _p(g), _p(dla), _p(dlb), _p(dlh0), B, T, d)
    return dla, dlb, dlh0


def linear_fwd(a, b, h0):
    """h (B,T,d) of h_t = a_t h_{t-1} + b_t (linear space, a of either sign)."""
    a, b, h0 = _f64(a), _f64(b), _f64(h0)
    B, T, d = a.shape
    assert b.shape == a.shape and h0.shape == (B, d)
    h = np.empty((B, T, d), np.float64)
    _load().oracle_linear_fwd(_p(a), _p(b), _p(h0), _p(h), B, T, d)
    return h


def linear_bwd(a, b, h0, dh):
    """(da, db, dh0) for L = sum(dh * h)."""
    a, b, h0, g = _f64(a), _f64(b), _f64(h0), _f64(dh)
    B, T, d = a.shape
    assert b.shape == a.shape and g.shape == a.shape and h0.shape == (B, d)
    da = np.empty_like(a)
    db = np.empty_like(a)
    dh0 = np.empty_like(h0)
    _load().oracle_linear_bwd(_p(a), _p(b), _p(h0), _p(g), _p(da), _p(db), _p(dh0), B, T, d)
    return da, db, dh0


def mingru_fwd(k, x, x0):
    """h (B,T,d) of the minGRU cell + scan from pre-activations k, x (B,T,d) and x0 (B,d)."""
    k, x, x0 = _f64(k), _f64(x), _f64(x0)
    B, T, d = k.shape
    assert x.shape == k.shape and x0.shape == (B, d)
    h = np.empty((B, T, d), np.float64)
    _load().oracle_mingru_fwd(_p(k), _p(x), _p(x0), _p(h), B, T, d)
    return h


def mingru_bwd(k, x, x0, dh):
    """(dk, dx, dx0) for L = sum(dh * h)."""
    k, x, x0, g = _f64(k), _f64(x), _f64(x0), _f64(dh)
    B, T, d = k.shape
    assert x.shape == k.shape and g.shape == k.shape and x0.shape == (B, d)
    dk = np.empty_like(k)
    dx = np.empty_like(k)
    dx0 = np.empty_like(x0)
    _load().oracle_mingru_bwd(_p(k), _p(x), _p(x0), _p(g), _p(dk), _p(dx), _p(dx0), B, T, d)
    return dk, dx, dx0


def _block_shapes(A, d, k):
    B, T, nb, k1, k2 = A.shape
    assert k1 == k and k2 == k and nb * k == d
    return B, T


def block_affine_fwd(A, b, h0, k):
    """h (B,T,d) of h_t = A_t h_{t-1} + b_t; A (B,T,d/k,k,k); h0 may be None (zeros)."""
    A64, b64 = _f64(A), _f64(b)
    B, T, d = b64.shape
    _block_shapes(A64, d, k)
    h064 = None if h0 is None else _f64(h0)
    h = np.empty((B, T, d), np.float64)
    _load().oracle_block_affine_fwd(_p(A64), _p(b64), _p(h064), _p(h), B, T, d, k)
    return h


def block_affine_bwd(A, b, h0, dh, k):
    """(dA, db, dh0) for L = sum(dh * h) of the block-affine scan."""
    A64, b64, g = _f64(A), _f64(b), _f64(dh)
    B, T, d = b64.shape
    _block_shapes(A64, d, k)
    h064 = None if h0 is None else _f64(h0)
    dA = np.empty_like(A64)
    db = np.empty_like(b64)
    dh0 = np.empty((B, d), np.float64)
    _load().oracle_block_affine_bwd(_p(A64), _p(b64), _p(h064), _p(g), _p(dA), _p(db), _p(dh0),
                                    B, T, d, k)
    return dA, db, dh0


def block_matrix_fwd(A, k):
    """P (B,T,d/k,k,k) with P_t = A_t P_{t-1}, P_0 = I."""
    A64 = _f64(A)
    B, T, nb = A64.shape[:3]
    d = nb * k
    _block_shapes(A64, d, k)
    P = np.empty_like(A64)
    _load().oracle_block_matrix_fwd(_p(A64), _p(P), B, T, d, k)
    return P


def block_matrix_bwd(A, dP, k):
    """dA for L = sum(dP * P) of the block cumulative product."""
    A64, g = _f64(A), _f64(dP)
    B, T, nb = A64.shape[:3]
    d = nb * k
    _block_shapes(A64, d, k)
    assert g.shape == A64.shape
    dA = np.empty_like(A64)
    _load().oracle_block_matrix_bwd(_p(A64), _p(g), _p(dA), B, T, d, k)
    return dA


def _givens_shapes(theta, s, d, k):
    B, T, nb, na = theta.shape
    assert nb * k == d and na == k * (k - 1) // 2 and s.shape == (B, T, nb)
    return B, T


def givens_fwd(theta, s, b, h0, k):
    """h (B,T,d) of h_t = sigmoid(s_t) R(theta_t) h_{t-1} + b_t (per block); h0 may be None."""
    theta, s, b = _f64(theta), _f64(s), _f64(b)
    h0 = None if h0 is None else _f64(h0)
    d = b.shape[2]
    B, T = _givens_shapes(theta, s, d, k)
    h = np.empty((B, T, d), np.float64)
    _load().oracle_givens_fwd(_p(theta), _p(s), _p(b), _p(h0), _p(h), B, T, d, k)
    return h


def givens_bwd(theta, s, b, h0, dh, k):
    """(dtheta, ds, db, dh0) for L = sum(dh * h)."""
    theta, s, b, g = _f64(theta), _f64(s), _f64(b), _f64(dh)
    h0 = None if h0 is None else _f64(h0)
    B, T, d = b.shape
    _givens_shapes(theta, s, d, k)
    dtheta = np.empty_like(theta)
    ds = np.empty_like(s)
    db = np.empty_like(b)
    dh0 = np.empty((B, d), np.float64)
    _load().oracle_givens_bwd(_p(theta), _p(s), _p(b), _p(h0), _p(g), _p(dtheta), _p(ds), _p(db), _p(dh0),
                              B, T, d, k)
    return dtheta, ds, db, dh0


def givens_matrix(theta, s, k):
    """A = sigmoid(s) R(theta) per block, as the Givens oracle forms it: (B,T,nb,k,k)."""
    theta, s = _f64(theta), _f64(s)
    B, T, nb, na = theta.shape
    eye = np.broadcast_to(np.eye(k), (B, T, nb, k, k)).copy()
    # P_t = A_t with h-columns: run the forward on unit vectors through the public loop
    out = np.empty((B, T, nb, k, k))
    for c in range(k):
        b0 = np.zeros((B, 1, nb * k))
        h0 = np.zeros((B, nb * k))
        h0[:, c::k] = 1.0
        for t in range(T):
            col = givens_fwd(theta[:, t:t + 1], s[:, t:t + 1], b0, h0, k)[:, 0]
            out[:, t, :, :, c] = col.reshape(B, nb, k)
    return out



def delta_fwd(q, k, v, beta, S0=None):
    """(o (B,T,dv), S_T (B,dv,dk)) of the delta rule; S0 (B,dv,dk) or None (zeros)."""
    q, k, v, beta = _f64(q), _f64(k), _f64(v), _f64(beta)
    S0 = None if S0 is None else _f64(S0)
    B, T, dk = k.shape
    dv = v.shape[2]
    assert q.shape == k.shape and v.shape[:2] == (B, T) and beta.shape == (B, T)
    assert S0 is None or S0.shape == (B, dv, dk)
    o = np.empty((B, T, dv), np.float64)
    ST = np.empty((B, dv, dk), np.float64)
    _load().oracle_delta_fwd(_p(q), _p(k), _p(v), _p(beta), _p(S0), _p(o), _p(ST), B, T, dk, dv)
    return o, ST
