"""C-ABI contract checks that need no GPU.

The library must load on a host without a GPU, export every function that
include/mgs.h declares, and reject bad arguments with the documented status
before any HIP call (so these run with fake, never-dereferenced pointers).
"""
import ctypes
import subprocess

import pytest

from scan_linear_rnns_amd import _lib

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3
BASE = 0x7F0000000000          # fake, 256-byte aligned device addresses (never dereferenced)


def fake(i, off=0):
    return ctypes.c_void_p(BASE + i * (1 << 32) + off)


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_exports_every_declared_symbol(lib):
    declared = _lib.declared_functions()
    assert len(declared) == 26, declared
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    missing = [n for n in declared if n not in exported]
    assert not missing, missing
    for name in declared:
        assert hasattr(lib, name)
        assert name in _lib.SIGNATURES


def test_version_and_strings(lib):
    assert lib.mgs_version() >= 100
    for s in range(5):
        assert _lib.status_string(s).startswith(("MGS_OK", "MGS_ERR"))
    assert "unknown" in _lib.status_string(99)
    assert lib.mgs_last_hip_error() == 0


def _size(lib, fn, *dims):
    out = ctypes.c_size_t(0)
    st = getattr(lib, fn)(*dims, ctypes.byref(out))
    return st, out.value


def test_workspace_queries(lib):
    for shape in ((2, 64, 16), (16, 1024, 64)):   # one layout serves both elementwise scans
        assert _size(lib, "mgs_scan_linear_workspace_size", *shape) == \
            _size(lib, "mgs_scan_log_workspace_size", *shape)
    st, small = _size(lib, "mgs_scan_log_workspace_size", 2, 64, 16)
    assert st == OK and small >= 256
    st, big = _size(lib, "mgs_scan_log_workspace_size", 16, 1024, 64)
    assert st == OK and big > small
    assert _size(lib, "mgs_scan_log_workspace_size", -1, 4, 4)[0] == INVALID
    assert lib.mgs_scan_log_workspace_size(2, 3, 4, None) == INVALID
    assert _size(lib, "mgs_scan_log_workspace_size", 1 << 20, 1 << 10, 1 << 10)[0] == UNSUPPORTED
    for fn in ("mgs_block_affine_scan_workspace_size", "mgs_block_matrix_scan_workspace_size"):
        st, b1 = _size(lib, fn, 128, 64, 64, 8)
        assert st == OK and b1 >= 256
        st, b2 = _size(lib, fn, 16, 1024, 64, 8)
        assert st == OK and b2 > 256
        assert _size(lib, fn, 2, 4, 12, 8)[0] == INVALID       # d % k != 0
        for k in (1, 2, 4, 8, 16):                             # the envelope
            st, bk = _size(lib, fn, 16, 1024, 64, k)
            assert st == OK and bk > 256, k
        assert _size(lib, fn, 2, 4, 12, 6)[0] == UNSUPPORTED   # k outside the envelope
        assert _size(lib, fn, 2, 4, 64, 32)[0] == UNSUPPORTED
        assert _size(lib, fn, 2, 4, 16, 0)[0] == INVALID
        assert _size(lib, fn, 1 << 16, 1 << 10, 64, 8)[0] == UNSUPPORTED


@pytest.mark.parametrize("op", ["log", "linear", "mingru"])
def test_elementwise_fwd_validation(lib, op):
    B, T, d = 2, 8, 16
    ws = fake(9)
    fn = getattr(lib, f"mgs_scan_{op}_fwd")
    args = lambda la=fake(0), lb=fake(1), lh0=fake(2), h=fake(3), B=B, T=T, d=d, ws=ws, nbytes=1 << 20: \
        fn(la, lb, lh0, h, B, T, d, ws, nbytes, None)
    assert args(la=None) == INVALID
    assert args(h=None) == INVALID
    assert args(lh0=None) == INVALID
    assert args(B=-1) == INVALID
    assert args(h=fake(0)) == INVALID                       # output aliases an input
    assert args(h=fake(0, 4 * B * T * d - 16)) == INVALID   # partial overlap
    assert args(lb=fake(1, 4)) == INVALID                   # misaligned
    assert args(ws=None) == WORKSPACE
    assert args(nbytes=8) == WORKSPACE
    assert args(B=0, la=None, lb=None, lh0=None, h=None) == OK   # empty: nothing to do, no HIP call
    assert args(T=0, la=None, lb=None, h=None) == OK


@pytest.mark.parametrize("op", ["log", "linear", "mingru"])
def test_elementwise_bwd_validation(lib, op):
    B, T, d = 2, 8, 16
    fn = getattr(lib, f"mgs_scan_{op}_bwd")
    call = lambda dla=fake(4), dlh0=fake(6), ws=fake(9), nbytes=1 << 20, B=B: \
        fn(fake(0), fake(1), fake(2), fake(3), dla, fake(5), dlh0, B, T, d, ws, nbytes, 1, None)
    assert call(dla=None) == INVALID
    assert call(dlh0=None) == INVALID
    assert call(dla=fake(3)) == INVALID                      # dlog_a aliases dh
    assert call(dla=fake(5)) == INVALID                      # two outputs overlap
    assert call(ws=None) == WORKSPACE
    assert call(nbytes=16) == WORKSPACE
    assert call(B=-3) == INVALID


def test_block_validation(lib):
    B, T, d, k = 2, 8, 16, 8
    fwd = lambda A=fake(0), b=fake(1), h0=fake(2), h=fake(3), k=k, d=d, nbytes=1 << 20, ws=fake(9): \
        lib.mgs_block_affine_scan_fwd(A, b, h0, h, B, T, d, k, ws, nbytes, None)
    assert fwd(A=None) == INVALID
    assert fwd(b=None) == INVALID
    assert fwd(h=fake(1)) == INVALID
    assert fwd(k=32, d=64) == UNSUPPORTED
    assert fwd(k=3, d=12) == UNSUPPORTED
    assert fwd(d=12) == INVALID
    assert fwd(nbytes=0) == WORKSPACE
    assert fwd(ws=fake(9, 8)) == INVALID                    # misaligned workspace
    bwd = lambda h=fake(3), dA=fake(5), dh0=fake(7), nbytes=1 << 20: lib.mgs_block_affine_scan_bwd(
        fake(0), None, None, h, fake(4), dA, fake(6), dh0, B, T, d, k, fake(9), nbytes, None)
    assert bwd(h=None) == INVALID
    assert bwd(dA=fake(0)) == INVALID
    assert bwd(dh0=None) == INVALID
    assert bwd(nbytes=1) == WORKSPACE
    mf = lambda P=fake(1), k=k, d=d, nbytes=1 << 20: lib.mgs_block_matrix_scan_fwd(fake(0), P, B, T, d, k,
                                                                                  fake(9), nbytes, None)
    assert mf(P=None) == INVALID
    assert mf(P=fake(0)) == INVALID
    assert mf(k=32, d=64) == UNSUPPORTED
    assert mf(nbytes=2) == WORKSPACE
    mb = lambda dP=fake(2), dA=fake(3), nbytes=1 << 20: lib.mgs_block_matrix_scan_bwd(
        fake(0), dP, dA, B, T, d, k, fake(9), nbytes, 1, None)
    assert mb(dP=None) == INVALID
    assert mb(dA=fake(2)) == INVALID
    assert mb(dA=fake(0)) == INVALID
    assert mb(nbytes=3) == WORKSPACE


def test_givens_validation(lib):
    B, T, d, k = 2, 8, 16, 8
    st, nb = _size(lib, "mgs_givens_scan_workspace_size", B, T, d, k)
    assert st == OK and (st, nb) == _size(lib, "mgs_block_affine_scan_workspace_size", B, T, d, k)
    assert _size(lib, "mgs_givens_scan_workspace_size", B, T, 16, 4)[0] == UNSUPPORTED
    fwd = lambda th=fake(0), s=fake(1), h=fake(3), k=k, nbytes=1 << 20: lib.mgs_givens_scan_fwd(
        th, s, fake(2), None, h, B, T, d, k, fake(9), nbytes, None)
    assert fwd(th=None) == INVALID
    assert fwd(s=None) == INVALID
    assert fwd(h=fake(1)) == INVALID                        # output aliases the gate
    assert fwd(k=4) == UNSUPPORTED
    assert fwd(nbytes=0) == WORKSPACE
    bwd = lambda dth=fake(5), ds=fake(6), nbytes=1 << 20: lib.mgs_givens_scan_bwd(
        fake(0), fake(1), None, fake(3), fake(4), dth, ds, fake(7), fake(8), B, T, d, k, fake(9), nbytes, None)
    assert bwd(dth=None) == INVALID
    assert bwd(ds=fake(5)) == INVALID                       # two outputs overlap
    assert bwd(dth=fake(0)) == INVALID                      # d theta aliases theta
    assert bwd(nbytes=4) == WORKSPACE


def test_workspace_check_validation(lib):
    assert lib.mgs_workspace_check(None, None, None) == INVALID
    assert lib.mgs_workspace_set_waits(None, 0, 0, None) == INVALID


def test_delta_validation(lib):
    B, T, d = 2, 100, 64
    st, nb = _size(lib, "mgs_delta_workspace_size", B, T, d)
    assert st == OK and nb >= 256 + B * 2 * 3 * 64 * 64 * 4     # two chunks of 64 steps
    assert _size(lib, "mgs_delta_workspace_size", B, T, 32)[0] == UNSUPPORTED
    assert _size(lib, "mgs_delta_workspace_size", -1, T, d)[0] == INVALID
    fwd = lambda q=fake(0), k=fake(1), v=fake(2), beta=fake(3), S0=None, o=fake(5), ST=fake(6), d=d, T=T, \
        ws=fake(9), nbytes=1 << 24: lib.mgs_delta_fwd(q, k, v, beta, S0, o, ST, B, T, d, ws, nbytes, None)
    assert fwd(q=None) == INVALID
    assert fwd(beta=None) == INVALID
    assert fwd(o=None) == INVALID
    assert fwd(o=fake(1)) == INVALID                        # output aliases k
    assert fwd(ST=fake(5, 1024)) == INVALID                 # the two outputs overlap
    assert fwd(S0=fake(4, 8)) == INVALID                    # misaligned
    assert fwd(d=48) == UNSUPPORTED
    assert fwd(ws=None) == WORKSPACE
    assert fwd(nbytes=1024) == WORKSPACE
    assert fwd(T=0, ST=None) == OK                          # nothing to do, no HIP call


# Sizes whose products overflow int64 (or wrap to 0): each must be refused as out of
# envelope before any HIP call, never accepted as an empty no-op.
OVERFLOWING_ELEM = [(1, 1 << 40, 1 << 24),          # B*T*d = 2^64: wraps to exactly 0
                    (1 << 21, 1 << 21, 1 << 22),     # 2^64 again, spread over the three sizes
                    (3, (1 << 62) // 3 + 1, 4),      # signed overflow of a product
                    (1, 1 << 31, 1),                 # one dimension past the envelope
                    (1 << 16, 1 << 16, 1)]           # 2^32 elements, no int64 overflow


@pytest.mark.parametrize("B,T,d", OVERFLOWING_ELEM)
@pytest.mark.parametrize("op", ["log", "linear", "mingru"])
def test_elementwise_overflowing_sizes(lib, op, B, T, d):
    assert _size(lib, f"mgs_scan_{op}_workspace_size", B, T, d)[0] == UNSUPPORTED
    fwd = getattr(lib, f"mgs_scan_{op}_fwd")
    assert fwd(fake(0), fake(1), fake(2), fake(3), B, T, d, fake(9), 1 << 20, None) == UNSUPPORTED
    bwd = getattr(lib, f"mgs_scan_{op}_bwd")
    assert bwd(fake(0), fake(1), fake(2), fake(3), fake(4), fake(5), fake(6), B, T, d, fake(9), 1 << 20, 1,
               None) == UNSUPPORTED


OVERFLOWING_BLOCK = [(1, 1 << 40, 1 << 24, 8),      # B*T*d*k = 2^67; B*T*d alone wraps to 0
                     (1, 1 << 37, 1 << 24, 8),      # B*T*d*k = 2^64: wraps to exactly 0
                     (1 << 20, 1 << 20, 1 << 24, 16),
                     (1, 1 << 28, 64, 8)]           # 2^37 elements of A, no int64 overflow


@pytest.mark.parametrize("B,T,d,k", OVERFLOWING_BLOCK)
def test_block_overflowing_sizes(lib, B, T, d, k):
    for fn in ("mgs_block_affine_scan_workspace_size", "mgs_block_matrix_scan_workspace_size"):
        assert _size(lib, fn, B, T, d, k)[0] == UNSUPPORTED
    assert lib.mgs_block_affine_scan_fwd(fake(0), fake(1), None, fake(3), B, T, d, k, fake(9), 1 << 20,
                                         None) == UNSUPPORTED
    assert lib.mgs_block_affine_scan_bwd(fake(0), None, None, fake(3), fake(4), fake(5), fake(6), fake(7),
                                         B, T, d, k, fake(9), 1 << 20, None) == UNSUPPORTED
    assert lib.mgs_block_matrix_scan_fwd(fake(0), fake(1), B, T, d, k, fake(9), 1 << 20, None) == UNSUPPORTED
    assert lib.mgs_block_matrix_scan_bwd(fake(0), fake(1), fake(2), B, T, d, k, fake(9), 1 << 20, 1,
                                         None) == UNSUPPORTED
    if k == 8:
        assert _size(lib, "mgs_givens_scan_workspace_size", B, T, d, k)[0] == UNSUPPORTED
        assert lib.mgs_givens_scan_fwd(fake(0), fake(1), fake(2), None, fake(3), B, T, d, k, fake(9), 1 << 20,
                                       None) == UNSUPPORTED
        assert lib.mgs_givens_scan_bwd(fake(0), fake(1), None, fake(3), fake(4), fake(5), fake(6), fake(7),
                                       fake(8), B, T, d, k, fake(9), 1 << 20, None) == UNSUPPORTED


@pytest.mark.parametrize("B,T", [(1, 1 << 58), (1 << 52, 1 << 10), (1 << 20, 1 << 20), (1 << 20, 0)])
def test_delta_overflowing_sizes(lib, B, T):
    # (B,T,64) or the (B,64,64) state past 2^31 elements, with and without int64 wrap-around
    assert _size(lib, "mgs_delta_workspace_size", B, T, 64)[0] == UNSUPPORTED
    assert lib.mgs_delta_fwd(fake(0), fake(1), fake(2), fake(3), None, fake(5), fake(6), B, T, 64, fake(9),
                             1 << 24, None) == UNSUPPORTED


def test_empty_tensors_are_valid(lib):
    # a size of 0 is an empty tensor (documented): nothing to compute, no HIP call
    assert _size(lib, "mgs_scan_log_workspace_size", 0, 1 << 40, 16) == (UNSUPPORTED, 0)
    assert _size(lib, "mgs_scan_log_workspace_size", 0, 64, 16) == (OK, 256)
    assert _size(lib, "mgs_block_affine_scan_workspace_size", 4, 0, 64, 8) == (OK, 256)
    assert lib.mgs_block_affine_scan_fwd(None, None, None, None, 4, 0, 64, 8, None, 0, None) == OK
    assert lib.mgs_block_matrix_scan_fwd(None, None, 0, 16, 64, 8, None, 0, None) == OK


def test_noalloc_validation(lib):
    """The entry point that allocates nothing validates like the forward it
    mirrors and refuses shapes beyond its scratch before any HIP call."""
    B, T, d, k = 2, 8, 16, 8
    f = lambda A=fake(0), b=fake(1), h0=None, h=fake(3), B=B, T=T, d=d, k=k: \
        lib.mgs_block_affine_scan_fwd_noalloc(A, b, h0, h, B, T, d, k, None)
    assert f(A=None) == INVALID
    assert f(h=None) == INVALID
    assert f(h=fake(1)) == INVALID                 # output aliases b
    assert f(b=fake(1, 4)) == INVALID              # misaligned
    assert f(d=12) == INVALID                      # d % k != 0
    assert f(k=3, d=12) == UNSUPPORTED
    assert f(B=-1) == INVALID
    assert f(T=0, A=None, b=None, h=None) == OK    # empty: nothing to do
    assert f(B=1, T=1 << 40, d=1 << 24) == UNSUPPORTED   # overflowing sizes
    assert f(B=4097, T=8, d=64) == UNSUPPORTED     # B*d past the scratch's zero region (262144)
    assert f(B=16, T=1 << 16, d=64) == UNSUPPORTED  # look-back words past the scratch
    assert f(B=16, T=24449, d=64) == UNSUPPORTED     # just past the documented limit at 128 chains
