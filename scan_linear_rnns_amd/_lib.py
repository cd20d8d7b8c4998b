"""ctypes loader for libmgs.so (the C ABI in include/mgs.h).

Argument marshalling only: every computation happens in the HIP kernels behind
the C ABI.  If the library is missing this module raises; there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("MGS_LIBRARY", os.path.join(HERE, "libmgs.so"))
HEADER = os.path.join(os.path.dirname(HERE), "include", "mgs.h")

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t
_INT = ctypes.c_int

SIGNATURES = {
    "mgs_version": ([], _INT),
    "mgs_status_string": ([_INT], ctypes.c_char_p),
    "mgs_last_hip_error": ([], _INT),
    "mgs_workspace_check": ([_P, _P, ctypes.POINTER(_INT)], _INT),
    "mgs_workspace_set_waits": ([_P, ctypes.c_uint, _INT, _P], _INT),
    "mgs_scan_log_workspace_size": ([_I64, _I64, _I64, ctypes.POINTER(_SZ)], _INT),
    "mgs_scan_log_fwd": ([_P, _P, _P, _P, _I64, _I64, _I64, _P, _SZ, _P], _INT),
    "mgs_scan_log_bwd": ([_P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _P, _SZ, _INT, _P], _INT),
    "mgs_scan_mingru_workspace_size": ([_I64, _I64, _I64, ctypes.POINTER(_SZ)], _INT),
    "mgs_scan_mingru_fwd": ([_P, _P, _P, _P, _I64, _I64, _I64, _P, _SZ, _P], _INT),
    "mgs_scan_mingru_bwd": ([_P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _P, _SZ, _INT, _P], _INT),
    "mgs_scan_linear_workspace_size": ([_I64, _I64, _I64, ctypes.POINTER(_SZ)], _INT),
    "mgs_scan_linear_fwd": ([_P, _P, _P, _P, _I64, _I64, _I64, _P, _SZ, _P], _INT),
    "mgs_scan_linear_bwd": ([_P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _P, _SZ, _INT, _P], _INT),
    "mgs_block_affine_scan_workspace_size": ([_I64, _I64, _I64, _I64, ctypes.POINTER(_SZ)], _INT),
    "mgs_block_affine_scan_fwd": ([_P, _P, _P, _P, _I64, _I64, _I64, _I64, _P, _SZ, _P], _INT),
    "mgs_block_affine_scan_fwd_noalloc": ([_P, _P, _P, _P, _I64, _I64, _I64, _I64, _P], _INT),
    "mgs_block_affine_scan_bwd": ([_P, _P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _P, _SZ, _P],
                                  _INT),
    "mgs_givens_scan_workspace_size": ([_I64, _I64, _I64, _I64, ctypes.POINTER(_SZ)], _INT),
    "mgs_givens_scan_fwd": ([_P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _P, _SZ, _P], _INT),
    "mgs_givens_scan_bwd": ([_P, _P, _P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _P, _SZ, _P], _INT),
    "mgs_block_matrix_scan_workspace_size": ([_I64, _I64, _I64, _I64, ctypes.POINTER(_SZ)], _INT),
    "mgs_block_matrix_scan_fwd": ([_P, _P, _I64, _I64, _I64, _I64, _P, _SZ, _P], _INT),
    "mgs_block_matrix_scan_bwd": ([_P, _P, _P, _I64, _I64, _I64, _I64, _P, _SZ, _INT, _P], _INT),
    "mgs_delta_workspace_size": ([_I64, _I64, _I64, ctypes.POINTER(_SZ)], _INT),
    "mgs_delta_fwd": ([_P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _P, _SZ, _P], _INT),
}

_lib = None


class MgsError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = status_string(status)
        if status == 4:  # MGS_ERR_HIP
            msg += f" (hipError_t {load().mgs_last_hip_error()})"
        super().__init__(f"{where}: {msg}")


def load():
    """Loads libmgs.so once; raises if it is missing (build it first)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libmgs.so not found at {LIB_PATH}: build it with "
                               "`python -m scan_linear_rnns_amd.build` (no CPU fallback exists)")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = res
        _lib = lib
    return _lib


def status_string(status: int) -> str:
    return load().mgs_status_string(int(status)).decode()


def check(status: int, where: str) -> None:
    if status != 0:
        raise MgsError(status, where)


def declared_functions():
    """Names of every function declared in include/mgs.h."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mgs_[a-z0-9_]+)\s*\(", text)))
