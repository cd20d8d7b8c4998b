"""scan_linear_rnns_amd -- the minGRU scan engine on AMD MI355X (gfx950).

Thin Python binding over the C ABI of libmgs.so (include/mgs.h).  Each
function below carries the name of the C entry point it calls and only
marshals arguments: torch supplies device memory and the current HIP stream;
every step of every scan runs in the library's HIP kernels.  There is no CPU
or PyTorch fallback: without the built library (or a GPU) these calls raise.

Ops (see include/mgs.h for the definitions and their sources on the pages):
  * mgs_scan_log_fwd / mgs_scan_log_bwd                 log-space minGRU scan
  * mgs_scan_mingru_fwd / mgs_scan_mingru_bwd           minGRU cell fused ahead of the log-space scan
  * mgs_scan_linear_fwd / mgs_scan_linear_bwd           linear-space scan, signed gates
  * mgs_block_affine_scan_fwd / mgs_block_affine_scan_bwd   h_t = A_t h_{t-1} + b_t
  * mgs_givens_scan_fwd / mgs_givens_scan_bwd           same, A_t = sigmoid(s_t) R(theta_t) formed in-kernel
  * mgs_block_matrix_scan_fwd / mgs_block_matrix_scan_bwd   P_t = A_t P_{t-1}
  * mgs_delta_fwd                                       delta rule (DeltaNet), chunked WY forward
"""
from __future__ import annotations

import ctypes

from . import _lib
from ._lib import MgsError, check, declared_functions, load, status_string  # noqa: F401

__all__ = [
    "MgsError", "load", "workspace", "mgs_workspace_check", "mgs_workspace_set_waits",
    "mgs_scan_log_workspace_size", "mgs_scan_log_fwd", "mgs_scan_log_bwd",
    "mgs_scan_mingru_workspace_size", "mgs_scan_mingru_fwd", "mgs_scan_mingru_bwd",
    "mgs_scan_linear_workspace_size", "mgs_scan_linear_fwd", "mgs_scan_linear_bwd",
    "mgs_block_affine_scan_workspace_size", "mgs_block_affine_scan_fwd", "mgs_block_affine_scan_bwd",
    "mgs_givens_scan_workspace_size", "mgs_givens_scan_fwd", "mgs_givens_scan_bwd",
    "mgs_block_matrix_scan_workspace_size", "mgs_block_matrix_scan_fwd", "mgs_block_matrix_scan_bwd",
    "mgs_delta_workspace_size", "mgs_delta_fwd",
]


def _ptr(t):
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check_tensor(name, t, shape, device=None):
    import torch
    if t is None:
        raise ValueError(f"{name} is required")
    if t.dtype != torch.float32:
        raise TypeError(f"{name} must be float32, got {t.dtype}")
    if not t.is_cuda:
        raise TypeError(f"{name} must be a GPU tensor (no CPU path exists)")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _size(fn, *dims):
    out = ctypes.c_size_t(0)
    check(getattr(load(), fn)(*[ctypes.c_int64(int(x)) for x in dims], ctypes.byref(out)), fn)
    return int(out.value)


def mgs_scan_log_workspace_size(B, T, d):
    return _size("mgs_scan_log_workspace_size", B, T, d)


def mgs_scan_mingru_workspace_size(B, T, d):
    return _size("mgs_scan_mingru_workspace_size", B, T, d)


def mgs_scan_linear_workspace_size(B, T, d):
    return _size("mgs_scan_linear_workspace_size", B, T, d)


def mgs_block_affine_scan_workspace_size(B, T, d, k):
    return _size("mgs_block_affine_scan_workspace_size", B, T, d, k)


def mgs_block_matrix_scan_workspace_size(B, T, d, k):
    return _size("mgs_block_matrix_scan_workspace_size", B, T, d, k)


def workspace(nbytes, device):
    """A zero-filled workspace of nbytes on device (zero-fill is required before first use)."""
    import torch
    return torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def mgs_workspace_check(ws, stream=None):
    """Device-side error flags of a workspace (0 = clean); clears them."""
    flags = ctypes.c_int(0)
    check(load().mgs_workspace_check(_ptr(ws), _stream(stream), ctypes.byref(flags)), "mgs_workspace_check")
    return int(flags.value)


def mgs_workspace_set_waits(ws, spin_limit=0, fail_waits=False, stream=None):
    """Failure-path test hook: the look-back waits' poll limit (0 = built-in) and,
    with fail_waits, waits that can never succeed (results then invalid)."""
    check(load().mgs_workspace_set_waits(_ptr(ws), int(spin_limit), int(bool(fail_waits)), _stream(stream)),
          "mgs_workspace_set_waits")


# --------------------------------------------------------------- log scan

def mgs_scan_log_fwd(log_a, log_b, log_h0, h=None, ws=None, stream=None):
    """h (B,T,d) of the log-space scan; returns (h, ws)."""
    import torch
    B, T, d = log_a.shape
    dev = log_a.device
    _check_tensor("log_a", log_a, (B, T, d))
    _check_tensor("log_b", log_b, (B, T, d), dev)
    _check_tensor("log_h0", log_h0, (B, d), dev)
    if h is None:
        h = torch.empty((B, T, d), dtype=torch.float32, device=dev)
    _check_tensor("h", h, (B, T, d), dev)
    if ws is None:
        ws = workspace(mgs_scan_log_workspace_size(B, T, d), dev)
    check(load().mgs_scan_log_fwd(_ptr(log_a), _ptr(log_b), _ptr(log_h0), _ptr(h), B, T, d,
                                  _ptr(ws), ws.numel(), _stream(stream)), "mgs_scan_log_fwd")
    return h, ws


def mgs_scan_log_bwd(log_a, log_b, log_h0, dh, ws=None, fwd_state_valid=False, out=None, stream=None):
    """(dlog_a, dlog_b, dlog_h0) for L = sum(dh * h)."""
    import torch
    B, T, d = log_a.shape
    dev = log_a.device
    _check_tensor("log_a", log_a, (B, T, d))
    _check_tensor("log_b", log_b, (B, T, d), dev)
    _check_tensor("log_h0", log_h0, (B, d), dev)
    _check_tensor("dh", dh, (B, T, d), dev)
    if out is None:
        out = (torch.empty((B, T, d), dtype=torch.float32, device=dev),
               torch.empty((B, T, d), dtype=torch.float32, device=dev),
               torch.empty((B, d), dtype=torch.float32, device=dev))
    dla, dlb, dlh0 = out
    if ws is None:
        ws = workspace(mgs_scan_log_workspace_size(B, T, d), dev)
        fwd_state_valid = False
    check(load().mgs_scan_log_bwd(_ptr(log_a), _ptr(log_b), _ptr(log_h0), _ptr(dh), _ptr(dla), _ptr(dlb),
                                  _ptr(dlh0), B, T, d, _ptr(ws), ws.numel(), int(bool(fwd_state_valid)),
                                  _stream(stream)), "mgs_scan_log_bwd")
    return dla, dlb, dlh0


# ------------------------------------------ minGRU cell + log-space scan

def _elem_fwd(fn, names, x1, x2, x0, h, ws, stream, size_fn):
    import torch
    B, T, d = x1.shape
    dev = x1.device
    _check_tensor(names[0], x1, (B, T, d))
    _check_tensor(names[1], x2, (B, T, d), dev)
    _check_tensor(names[2], x0, (B, d), dev)
    if h is None:
        h = torch.empty((B, T, d), dtype=torch.float32, device=dev)
    _check_tensor("h", h, (B, T, d), dev)
    if ws is None:
        ws = workspace(size_fn(B, T, d), dev)
    check(getattr(load(), fn)(_ptr(x1), _ptr(x2), _ptr(x0), _ptr(h), B, T, d, _ptr(ws), ws.numel(),
                              _stream(stream)), fn)
    return h, ws


def _elem_bwd(fn, names, x1, x2, x0, dh, ws, fwd_state_valid, out, stream, size_fn):
    import torch
    B, T, d = x1.shape
    dev = x1.device
    _check_tensor(names[0], x1, (B, T, d))
    _check_tensor(names[1], x2, (B, T, d), dev)
    _check_tensor(names[2], x0, (B, d), dev)
    _check_tensor("dh", dh, (B, T, d), dev)
    if out is None:
        out = (torch.empty((B, T, d), dtype=torch.float32, device=dev),
               torch.empty((B, T, d), dtype=torch.float32, device=dev),
               torch.empty((B, d), dtype=torch.float32, device=dev))
    d1, d2, d0 = out
    if ws is None:
        ws = workspace(size_fn(B, T, d), dev)
        fwd_state_valid = False
    check(getattr(load(), fn)(_ptr(x1), _ptr(x2), _ptr(x0), _ptr(dh), _ptr(d1), _ptr(d2), _ptr(d0),
                              B, T, d, _ptr(ws), ws.numel(), int(bool(fwd_state_valid)), _stream(stream)), fn)
    return d1, d2, d0


def mgs_scan_mingru_fwd(k, x, x0, h=None, ws=None, stream=None):
    """h (B,T,d) of the minGRU cell + log-space scan from pre-activations; returns (h, ws)."""
    return _elem_fwd("mgs_scan_mingru_fwd", ("k", "x", "x0"), k, x, x0, h, ws, stream,
                     mgs_scan_mingru_workspace_size)


def mgs_scan_mingru_bwd(k, x, x0, dh, ws=None, fwd_state_valid=False, out=None, stream=None):
    """(dk, dx, dx0) for L = sum(dh * h)."""
    return _elem_bwd("mgs_scan_mingru_bwd", ("k", "x", "x0"), k, x, x0, dh, ws, fwd_state_valid, out,
                     stream, mgs_scan_mingru_workspace_size)


# ----------------------------------------------------- linear-space scan

def mgs_scan_linear_fwd(a, b, h0, h=None, ws=None, stream=None):
    """h (B,T,d) of h_t = a_t h_{t-1} + b_t (a of either sign); returns (h, ws)."""
    import torch
    B, T, d = a.shape
    dev = a.device
    _check_tensor("a", a, (B, T, d))
    _check_tensor("b", b, (B, T, d), dev)
    _check_tensor("h0", h0, (B, d), dev)
    if h is None:
        h = torch.empty((B, T, d), dtype=torch.float32, device=dev)
    _check_tensor("h", h, (B, T, d), dev)
    if ws is None:
        ws = workspace(mgs_scan_linear_workspace_size(B, T, d), dev)
    check(load().mgs_scan_linear_fwd(_ptr(a), _ptr(b), _ptr(h0), _ptr(h), B, T, d,
                                     _ptr(ws), ws.numel(), _stream(stream)), "mgs_scan_linear_fwd")
    return h, ws


def mgs_scan_linear_bwd(a, b, h0, dh, ws=None, fwd_state_valid=False, out=None, stream=None):
    """(da, db, dh0) for L = sum(dh * h)."""
    import torch
    B, T, d = a.shape
    dev = a.device
    _check_tensor("a", a, (B, T, d))
    _check_tensor("b", b, (B, T, d), dev)
    _check_tensor("h0", h0, (B, d), dev)
    _check_tensor("dh", dh, (B, T, d), dev)
    if out is None:
        out = (torch.empty((B, T, d), dtype=torch.float32, device=dev),
               torch.empty((B, T, d), dtype=torch.float32, device=dev),
               torch.empty((B, d), dtype=torch.float32, device=dev))
    da, db, dh0 = out
    if ws is None:
        ws = workspace(mgs_scan_linear_workspace_size(B, T, d), dev)
        fwd_state_valid = False
    check(load().mgs_scan_linear_bwd(_ptr(a), _ptr(b), _ptr(h0), _ptr(dh), _ptr(da), _ptr(db), _ptr(dh0),
                                     B, T, d, _ptr(ws), ws.numel(), int(bool(fwd_state_valid)),
                                     _stream(stream)), "mgs_scan_linear_bwd")
    return da, db, dh0


# ---------------------------------------------------------- block-affine

def _block_dims(A, k):
    B, T, nb, k1, k2 = A.shape
    if k1 != k or k2 != k:
        raise ValueError(f"A must have trailing dims ({k},{k}), got {tuple(A.shape)}")
    return B, T, nb * k


def mgs_block_affine_scan_fwd(A, b, h0, k=8, h=None, ws=None, stream=None):
    """h (B,T,d) of h_t = A_t h_{t-1} + b_t; h0 may be None (zeros); returns (h, ws)."""
    import torch
    B, T, d = _block_dims(A, k)
    dev = A.device
    _check_tensor("A", A, (B, T, d // k, k, k))
    _check_tensor("b", b, (B, T, d), dev)
    if h0 is not None:
        _check_tensor("h0", h0, (B, d), dev)
    if h is None:
        h = torch.empty((B, T, d), dtype=torch.float32, device=dev)
    _check_tensor("h", h, (B, T, d), dev)
    if ws is None:
        ws = workspace(mgs_block_affine_scan_workspace_size(B, T, d, k), dev)
    check(load().mgs_block_affine_scan_fwd(_ptr(A), _ptr(b), _ptr(h0), _ptr(h), B, T, d, k, _ptr(ws),
                                           ws.numel(), _stream(stream)), "mgs_block_affine_scan_fwd")
    return h, ws


def mgs_block_affine_scan_fwd_noalloc(A, b, h0, k=8, h=None, stream=None):
    """mgs_block_affine_scan_fwd without a workspace (the library's own device
    scratch); returns h.  Pass a preallocated h to allocate nothing here either."""
    import torch
    B, T, d = _block_dims(A, k)
    dev = A.device
    _check_tensor("A", A, (B, T, d // k, k, k))
    _check_tensor("b", b, (B, T, d), dev)
    if h0 is not None:
        _check_tensor("h0", h0, (B, d), dev)
    if h is None:
        h = torch.empty((B, T, d), dtype=torch.float32, device=dev)
    _check_tensor("h", h, (B, T, d), dev)
    check(load().mgs_block_affine_scan_fwd_noalloc(_ptr(A), _ptr(b), _ptr(h0), _ptr(h), B, T, d, k,
                                                   _stream(stream)), "mgs_block_affine_scan_fwd_noalloc")
    return h


def mgs_block_affine_scan_bwd(A, b, h0, h, dh, k=8, ws=None, out=None, stream=None):
    """(dA, db, dh0) for L = sum(dh * h); h is the forward's output."""
    import torch
    B, T, d = _block_dims(A, k)
    dev = A.device
    _check_tensor("A", A, (B, T, d // k, k, k))
    if b is not None:
        _check_tensor("b", b, (B, T, d), dev)
    if h0 is not None:
        _check_tensor("h0", h0, (B, d), dev)
    _check_tensor("h", h, (B, T, d), dev)
    _check_tensor("dh", dh, (B, T, d), dev)
    if out is None:
        out = (torch.empty_like(A), torch.empty((B, T, d), dtype=torch.float32, device=dev),
               torch.empty((B, d), dtype=torch.float32, device=dev))
    dA, db, dh0 = out
    if ws is None:
        ws = workspace(mgs_block_affine_scan_workspace_size(B, T, d, k), dev)
    check(load().mgs_block_affine_scan_bwd(_ptr(A), _ptr(b), _ptr(h0), _ptr(h), _ptr(dh), _ptr(dA), _ptr(db),
                                           _ptr(dh0), B, T, d, k, _ptr(ws), ws.numel(), _stream(stream)),
          "mgs_block_affine_scan_bwd")
    return dA, db, dh0


# ---------------------------------------------- Givens angle-fused scan

def mgs_givens_scan_workspace_size(B, T, d, k):
    return _size("mgs_givens_scan_workspace_size", B, T, d, k)


def _givens_dims(theta, k):
    B, T, nb, na = theta.shape
    if na != k * (k - 1) // 2:
        raise ValueError(f"theta must have trailing dim {k * (k - 1) // 2}, got {tuple(theta.shape)}")
    return B, T, nb * k


def mgs_givens_scan_fwd(theta, s, b, h0, k=8, h=None, ws=None, stream=None):
    """h (B,T,d) of h_t = sigmoid(s_t) R(theta_t) h_{t-1} + b_t; h0 may be None; returns (h, ws)."""
    import torch
    B, T, d = _givens_dims(theta, k)
    dev = theta.device
    _check_tensor("theta", theta, tuple(theta.shape))
    _check_tensor("s", s, (B, T, d // k), dev)
    _check_tensor("b", b, (B, T, d), dev)
    if h0 is not None:
        _check_tensor("h0", h0, (B, d), dev)
    if h is None:
        h = torch.empty((B, T, d), dtype=torch.float32, device=dev)
    _check_tensor("h", h, (B, T, d), dev)
    if ws is None:
        ws = workspace(mgs_givens_scan_workspace_size(B, T, d, k), dev)
    check(load().mgs_givens_scan_fwd(_ptr(theta), _ptr(s), _ptr(b), _ptr(h0), _ptr(h), B, T, d, k, _ptr(ws),
                                     ws.numel(), _stream(stream)), "mgs_givens_scan_fwd")
    return h, ws


def mgs_givens_scan_bwd(theta, s, h0, h, dh, k=8, ws=None, out=None, stream=None):
    """(dtheta, ds, db, dh0) for L = sum(dh * h); h is the forward's output."""
    import torch
    B, T, d = _givens_dims(theta, k)
    dev = theta.device
    _check_tensor("theta", theta, tuple(theta.shape))
    _check_tensor("s", s, (B, T, d // k), dev)
    if h0 is not None:
        _check_tensor("h0", h0, (B, d), dev)
    _check_tensor("h", h, (B, T, d), dev)
    _check_tensor("dh", dh, (B, T, d), dev)
    if out is None:
        out = (torch.empty_like(theta), torch.empty_like(s), torch.empty((B, T, d), dtype=torch.float32, device=dev),
               torch.empty((B, d), dtype=torch.float32, device=dev))
    dth, ds, db, dh0 = out
    if ws is None:
        ws = workspace(mgs_givens_scan_workspace_size(B, T, d, k), dev)
    check(load().mgs_givens_scan_bwd(_ptr(theta), _ptr(s), _ptr(h0), _ptr(h), _ptr(dh), _ptr(dth), _ptr(ds),
                                     _ptr(db), _ptr(dh0), B, T, d, k, _ptr(ws), ws.numel(), _stream(stream)),
          "mgs_givens_scan_bwd")
    return dth, ds, db, dh0


# ------------------------------------------------- block cumulative product

def mgs_block_matrix_scan_fwd(A, k=8, P=None, ws=None, stream=None):
    """P (B,T,d/k,k,k) with P_t = A_t P_{t-1}, P_0 = I; returns (P, ws)."""
    import torch
    B, T, d = _block_dims(A, k)
    _check_tensor("A", A, (B, T, d // k, k, k))
    if P is None:
        P = torch.empty_like(A)
    _check_tensor("P", P, tuple(A.shape), A.device)
    if ws is None:
        ws = workspace(mgs_block_matrix_scan_workspace_size(B, T, d, k), A.device)
    check(load().mgs_block_matrix_scan_fwd(_ptr(A), _ptr(P), B, T, d, k, _ptr(ws), ws.numel(), _stream(stream)),
          "mgs_block_matrix_scan_fwd")
    return P, ws


def mgs_block_matrix_scan_bwd(A, dP, k=8, ws=None, fwd_state_valid=False, dA=None, stream=None):
    """dA for L = sum(dP * P).  Pass the forward's workspace with fwd_state_valid=True
    to reuse its saved chunk states; otherwise they are recomputed first."""
    import torch
    B, T, d = _block_dims(A, k)
    _check_tensor("A", A, (B, T, d // k, k, k))
    _check_tensor("dP", dP, tuple(A.shape), A.device)
    if dA is None:
        dA = torch.empty_like(A)
    if ws is None:
        ws = workspace(mgs_block_matrix_scan_workspace_size(B, T, d, k), A.device)
        fwd_state_valid = False
    check(load().mgs_block_matrix_scan_bwd(_ptr(A), _ptr(dP), _ptr(dA), B, T, d, k, _ptr(ws), ws.numel(),
                                           int(bool(fwd_state_valid)), _stream(stream)),
          "mgs_block_matrix_scan_bwd")
    return dA


# ------------------------------------------------------------ delta rule

def mgs_delta_workspace_size(B, T, d):
    return _size("mgs_delta_workspace_size", B, T, d)


def mgs_delta_fwd(q, k, v, beta, S0=None, o=None, ST=None, ws=None, want_state=True, stream=None):
    """(o (B,T,d), S_T (B,d,d) or None, ws) of S_t = S_{t-1} + beta_t (v_t - S_{t-1} k_t) k_t^T,
    o_t = S_t q_t; S0 (B,d,d) or None (zeros)."""
    import torch
    B, T, d = k.shape
    dev = k.device
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_tensor(name, t, (B, T, d), dev)
    _check_tensor("beta", beta, (B, T), dev)
    if S0 is not None:
        _check_tensor("S0", S0, (B, d, d), dev)
    if o is None:
        o = torch.empty((B, T, d), dtype=torch.float32, device=dev)
    _check_tensor("o", o, (B, T, d), dev)
    if ST is None and want_state:
        ST = torch.empty((B, d, d), dtype=torch.float32, device=dev)
    if ST is not None:
        _check_tensor("ST", ST, (B, d, d), dev)
    if ws is None:
        ws = workspace(mgs_delta_workspace_size(B, T, d), dev)
    check(load().mgs_delta_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(S0), _ptr(o), _ptr(ST), B, T, d,
                               _ptr(ws), ws.numel(), _stream(stream)), "mgs_delta_fwd")
    return o, ST, ws
