"""Seeded synthetic inputs for the minGRU scan engine.

This module is shared by the tests, the benchmark and the smoke check.  It
holds none of the scan arithmetic: it only draws random numbers and turns them
into the scan's inputs (gates, transition matrices, upstream gradients).

Recipes (numpy PCG64 ``default_rng(seed)``, every draw in float64, rounded
once to float32 at the end):

* Log-space minGRU scan (minGRU home page, introduction: the MinGRU gate of
  Feng et al.).  Draw k, x ~ N(0,1) of shape (B,T,d), then x0 ~ N(0,1) of shape
  (B,d), then dh ~ N(0,1) of shape (B,T,d).  With a = sigmoid(-k), z = 1 - a
  and g(x) = x + 0.5 for x >= 0, sigmoid(x) otherwise:
  log_a = log a, log_b = log(z * g(x)), log_h0 = log g(x0).  Logs are taken
  in closed form (log sigmoid(u) = -softplus(-u)) so nothing underflows.
* MinGRU cell fused ahead of the log-space scan: the same draws k, x, x0, dh,
  passed as pre-activations (the kernel forms log a, log b, log h0 itself).
* Linear-space scan with signed gates (linear_scan; SignedMinGRU's
  negative-eigenvalue gates on the home page).  Same draws as the log-space
  scan (k, x, x0, dh in that order); the MinGRU gate sigmoid(-k) in [0, 1] is
  stretched to a = 2 sigmoid(-k) - 1 in (-1, 1), b = (1 - sigmoid(-k)) g(x),
  h0 = g(x0).
* Delta rule (DeltaMinGRU on the home page, DeltaNet's recurrence): see
  delta_inputs.
* Block scans (GivensMinGRU on the home page; the Clements rectangular mesh of
  Givens rotations).  Draw s ~ N(0,1) of shape (B,T,nb), theta ~ U(-pi, pi) of
  shape (B,T,nb,k(k-1)/2), b ~ N(0,1) of shape (B,T,d), dh ~ N(0,1) of shape
  (B,T,d), and last (cumulative product only) dP ~ N(0,1) of shape
  (B,T,nb,k,k).  A_t = sigmoid(s_t) R(theta_t) where R is k layers of disjoint
  2x2 rotations: layer l acts on pairs (i, i+1) for i = l mod 2, l mod 2 + 2,
  ... < k-1; layers are applied in order (R = L_{k-1} ... L_0) and angles are
  consumed in (layer, pair) order.  Each rotation maps (x_i, x_j) to
  (cos t x_i - sin t x_j, sin t x_i + cos t x_j).  h0 = 0.

Tensors at the boundary's size limit (2^31 - 1 elements) are too large to draw
on the host, so device_log_inputs / device_block_inputs draw them on a GPU with
torch's seeded generator (Philox), one batch slice at a time, with the same
distributions: the log-space recipe above evaluated in float32; for the block
scans A_t = sigmoid(s_t) Q where Q is picked uniformly from a bank of 4096
Givens meshes R(theta) (theta ~ U(-pi, pi), numpy seed) and s, b, dh, dP are
N(0,1).
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Optional

import numpy as np


def _softplus(u):
    return np.logaddexp(0.0, u)


def _log_g(x):
    # g(x) = x + 0.5 (x >= 0), sigmoid(x) (x < 0); log sigmoid(x) = -softplus(-x)
    return np.where(x >= 0, np.log(np.maximum(x, 0.0) + 0.5), -_softplus(-x))


@dataclass
class LogInputs:
    log_a: np.ndarray   # (B,T,d) float32
    log_b: np.ndarray   # (B,T,d) float32
    log_h0: np.ndarray  # (B,d)   float32
    dh: np.ndarray      # (B,T,d) float32


def mingru_logs(k, x, x0):
    """(log a, log b, log h0) in float64 of the MinGRU gate recipe, from pre-activations."""
    k, x, x0 = (np.asarray(v, dtype=np.float64) for v in (k, x, x0))
    log_a = -_softplus(k)            # log sigmoid(-k)
    log_z = -_softplus(-k)           # log (1 - sigmoid(-k)) = log sigmoid(k)
    return log_a, log_z + _log_g(x), _log_g(x0)


def log_inputs(B: int, T: int, d: int, seed: int = 0) -> LogInputs:
    """MinGRU gate generator for the log-space scan (see module docstring)."""
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((B, T, d))
    x = rng.standard_normal((B, T, d))
    x0 = rng.standard_normal((B, d))
    dh = rng.standard_normal((B, T, d))
    log_a, log_b, log_h0 = mingru_logs(k, x, x0)
    f = np.float32
    return LogInputs(log_a.astype(f), log_b.astype(f), log_h0.astype(f), dh.astype(f))


@dataclass
class MinGRUInputs:
    k: np.ndarray       # (B,T,d) float32, gate pre-activation
    x: np.ndarray       # (B,T,d) float32, candidate pre-activation
    x0: np.ndarray      # (B,d)   float32, initial-state pre-activation
    dh: np.ndarray      # (B,T,d) float32


def mingru_inputs(B: int, T: int, d: int, seed: int = 0) -> MinGRUInputs:
    """The log-space scan's draws before the gate recipe (same seed, same values)."""
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((B, T, d))
    x = rng.standard_normal((B, T, d))
    x0 = rng.standard_normal((B, d))
    dh = rng.standard_normal((B, T, d))
    f = np.float32
    return MinGRUInputs(k.astype(f), x.astype(f), x0.astype(f), dh.astype(f))


@dataclass
class LinearInputs:
    a: np.ndarray       # (B,T,d) float32, in (-1, 1)
    b: np.ndarray       # (B,T,d) float32
    h0: np.ndarray      # (B,d)   float32
    dh: np.ndarray      # (B,T,d) float32


def linear_inputs(B: int, T: int, d: int, seed: int = 0) -> LinearInputs:
    """Signed-gate generator for the linear-space scan (see module docstring)."""
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((B, T, d))
    x = rng.standard_normal((B, T, d))
    x0 = rng.standard_normal((B, d))
    dh = rng.standard_normal((B, T, d))
    gate = np.exp(-_softplus(k))     # sigmoid(-k)
    a = 2.0 * gate - 1.0
    b = (1.0 - gate) * np.exp(_log_g(x))
    h0 = np.exp(_log_g(x0))
    f = np.float32
    return LinearInputs(a.astype(f), b.astype(f), h0.astype(f), dh.astype(f))


def n_angles(k: int) -> int:
    return k * (k - 1) // 2


def givens_mesh(theta: np.ndarray, k: int) -> np.ndarray:
    """R(theta) in float64 for theta of shape (..., k(k-1)/2): shape (..., k, k)."""
    theta = np.asarray(theta, dtype=np.float64)
    assert theta.shape[-1] == n_angles(k)
    lead = theta.shape[:-1]
    R = np.broadcast_to(np.eye(k), lead + (k, k)).copy()
    idx = 0
    for layer in range(k):
        for i in range(layer % 2, k - 1, 2):
            c = np.cos(theta[..., idx])[..., None]
            s = np.sin(theta[..., idx])[..., None]
            ri = R[..., i, :].copy()
            rj = R[..., i + 1, :].copy()
            R[..., i, :] = c * ri - s * rj
            R[..., i + 1, :] = s * ri + c * rj
            idx += 1
    assert idx == n_angles(k)
    return R


@dataclass
class BlockInputs:
    A: np.ndarray                    # (B,T,nb,k,k) float32
    b: np.ndarray                    # (B,T,d) float32
    h0: Optional[np.ndarray]         # (B,d) float32 or None (zeros)
    dh: np.ndarray                   # (B,T,d) float32
    dP: Optional[np.ndarray]         # (B,T,nb,k,k) float32 (cumulative product only)
    k: int
    theta: Optional[np.ndarray] = None  # (B,T,nb,k(k-1)/2) float32 angles (Givens angle-fused scan)
    s: Optional[np.ndarray] = None      # (B,T,nb) float32 gate pre-activations (Givens angle-fused scan)


def block_inputs(B: int, T: int, d: int, k: int = 8, seed: int = 0, *,
                 gate: bool = True, with_dP: bool = True,
                 h0: str = "zero", return_angles: bool = False) -> BlockInputs:
    """Gated Givens-mesh generator for the block scans (see module docstring).

    gate=False drops the sigmoid gate (pure rotations, used for the long-T
    orthogonality checks).  h0="zero" gives h0 = None (zeros, as in the
    Givens lab configuration); h0="normal" draws h0 ~ N(0,1) after dP.
    return_angles=True also returns theta and s rounded to float32 (the inputs
    of the Givens angle-fused scan, which forms A from them itself).
    """
    assert d % k == 0
    nb = d // k
    rng = np.random.default_rng(seed)
    s = rng.standard_normal((B, T, nb))
    theta = rng.uniform(-math.pi, math.pi, (B, T, nb, n_angles(k)))
    b = rng.standard_normal((B, T, d))
    dh = rng.standard_normal((B, T, d))
    dP = rng.standard_normal((B, T, nb, k, k)) if with_dP else None
    h0v = rng.standard_normal((B, d)) if h0 == "normal" else None
    R = givens_mesh(theta, k)
    if gate:
        A = (1.0 / (1.0 + np.exp(-s)))[..., None, None] * R
    else:
        A = R
    f = np.float32
    return BlockInputs(A.astype(f), b.astype(f), None if h0v is None else h0v.astype(f),
                       dh.astype(f), None if dP is None else dP.astype(f), k,
                       theta.astype(f) if return_angles else None, s.astype(f) if return_angles else None)


@dataclass
class DeltaInputs:
    q: np.ndarray       # (B,T,d) float32, unit rows
    k: np.ndarray       # (B,T,d) float32, unit rows
    v: np.ndarray       # (B,T,d) float32
    beta: np.ndarray    # (B,T)   float32, in (0, 1)
    S0: Optional[np.ndarray]  # (B,d,d) float32 or None (zeros)


def delta_inputs(B: int, T: int, d: int, seed: int = 0, *, s0: str = "zero") -> DeltaInputs:
    """Delta-rule generator (DeltaMinGRU on the home page; DeltaNet's
    normalisation): q, k, v ~ N(0,1) of shape (B,T,d) in that order, then
    u ~ N(0,1) of shape (B,T), then (s0="normal") S0 ~ N(0,1) of shape (B,d,d).
    q and k are scaled to unit L2 norm per step, beta = sigmoid(u)."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, T, d))
    k = rng.standard_normal((B, T, d))
    v = rng.standard_normal((B, T, d))
    u = rng.standard_normal((B, T))
    S0 = rng.standard_normal((B, d, d)) if s0 == "normal" else None
    q = q / np.linalg.norm(q, axis=-1, keepdims=True)
    k = k / np.linalg.norm(k, axis=-1, keepdims=True)
    beta = 1.0 / (1.0 + np.exp(-u))
    f = np.float32
    return DeltaInputs(q.astype(f), k.astype(f), v.astype(f), beta.astype(f),
                       None if S0 is None else S0.astype(f))


# The five workloads, by name (shapes from the pages' lab and long-T
# microbenchmark shapes, d = 64 and k = 8 from the Givens memory measurement).
CONFIGS = {
    "log_tiny":   dict(op="log", B=2, T=64, d=16),
    "log_lab":    dict(op="log", B=128, T=64, d=64),
    "log_longT":  dict(op="log", B=16, T=1024, d=64),
    "mingru_lab":   dict(op="mingru", B=128, T=64, d=64),
    "mingru_longT": dict(op="mingru", B=16, T=1024, d=64),
    "linear_lab":   dict(op="linear", B=128, T=64, d=64),
    "linear_longT": dict(op="linear", B=16, T=1024, d=64),
    "block_lab":  dict(op="block", B=128, T=64, d=64, k=8),
    "block_longT": dict(op="block", B=16, T=1024, d=64, k=8),
    "delta_lab":   dict(op="delta", B=128, T=64, d=64),
    "delta_longT": dict(op="delta", B=16, T=1024, d=64),
}


# ------------------------------------------------ inputs drawn on a device

def _device_gen(device, seed):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _slices(B, per_item, limit=1 << 27):
    """Batch ranges of at most `limit` elements (at least one item each)."""
    n = max(1, limit // max(1, per_item))
    return [(i, min(B, i + n)) for i in range(0, B, n)]


def _log_g_t(x):
    import torch
    import torch.nn.functional as F
    return torch.where(x >= 0, torch.log(x.clamp_min(0) + 0.5), -F.softplus(-x))


def device_log_inputs(B: int, T: int, d: int, device, seed: int = 0):
    """(log_a, log_b, log_h0, dh) as float32 tensors on `device` (the log-space
    recipe in float32, drawn a batch slice at a time to bound temporaries)."""
    import torch
    import torch.nn.functional as F
    g = _device_gen(device, seed)
    f32 = dict(dtype=torch.float32, device=device)
    la = torch.empty((B, T, d), **f32)
    lb = torch.empty((B, T, d), **f32)
    dh = torch.empty((B, T, d), **f32)
    for i, j in _slices(B, T * d):
        k = torch.randn((j - i, T, d), generator=g, **f32)
        la[i:j] = -F.softplus(k)
        lb[i:j] = -F.softplus(k.neg_())
        del k
        x = torch.randn((j - i, T, d), generator=g, **f32)
        lb[i:j] += _log_g_t(x)
        del x
    lh0 = _log_g_t(torch.randn((B, d), generator=g, **f32))
    for i, j in _slices(B, T * d):
        dh[i:j] = torch.randn((j - i, T, d), generator=g, **f32)
    return la, lb, lh0, dh


def mesh_bank(n: int, k: int, seed: int = 0) -> np.ndarray:
    """n Givens meshes R(theta), theta ~ U(-pi, pi): (n, k, k) float32."""
    rng = np.random.default_rng(seed)
    theta = rng.uniform(-math.pi, math.pi, (n, n_angles(k)))
    return givens_mesh(theta, k).astype(np.float32)


def device_block_inputs(B: int, T: int, d: int, k: int, device, seed: int = 0, *, with_b: bool = True,
                        with_dh: bool = True, with_dP: bool = False):
    """dict of float32 tensors on `device`: A (B,T,d/k,k,k) = sigmoid(s) Q_idx
    (Q from mesh_bank(4096, k, seed)) and, as asked, b and dh (B,T,d) and dP
    (like A), all N(0,1); drawn a batch slice at a time."""
    import torch
    assert d % k == 0
    nb = d // k
    g = _device_gen(device, seed)
    f32 = dict(dtype=torch.float32, device=device)
    bank = torch.from_numpy(mesh_bank(4096, k, seed)).to(device)
    A = torch.empty((B, T, nb, k, k), **f32)
    for i, j in _slices(B, T * d * k):
        idx = torch.randint(0, bank.shape[0], (j - i, T, nb), generator=g, device=device)
        s = torch.sigmoid(torch.randn((j - i, T, nb), generator=g, **f32))
        torch.mul(bank[idx], s[..., None, None], out=A[i:j])
        del idx, s
    out = dict(A=A)
    for name, want, shape in (("b", with_b, (T, d)), ("dh", with_dh, (T, d)), ("dP", with_dP, (T, nb, k, k))):
        if not want:
            continue
        x = torch.empty((B,) + shape, **f32)
        for i, j in _slices(B, math.prod(shape)):
            x[i:j] = torch.randn((j - i,) + shape, generator=g, **f32)
        out[name] = x
    return out
