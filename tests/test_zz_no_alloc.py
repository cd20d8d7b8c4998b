"""GPU check of mgs_block_affine_scan_fwd_noalloc, the block-affine forward
that allocates nothing (its workspace is the library's own device scratch),
called through the C ABI and compared with mgs_block_affine_scan_fwd on the
same inputs.

Both entry points run the same kernels on the same geometry (only the
workspace offsets differ), so their outputs must agree bit for bit; the
existing entry point is itself held to the oracle by the parity tests.  The
calls come in a row on one GPU, each smaller than the one before it, so the
scratch carries the previous call's words (an older launch tag, a different
layout) into every call after the first: the long-T workload with h0 = 0
(multi-tile, decoupled look-back), then a ragged shape with h0 drawn (several
tiles along T), then the lab shape (one tile along T).
"""
import ctypes

import numpy as np
import pytest
import torch

from synthetic import block_inputs
from tests.test_parity_gpu import say, to_dev

pytestmark = pytest.mark.gpu

P = lambda x: ctypes.c_void_p(0 if x is None else x.data_ptr())


def _existing(lib, A, b, h0, B, T, d, k, stream):
    import scan_linear_rnns_amd as mgs
    nbytes = mgs.mgs_block_affine_scan_workspace_size(B, T, d, k)
    ws = mgs.workspace(nbytes, A.device)
    h = torch.empty((B, T, d), dtype=torch.float32, device=A.device)
    rc = lib.mgs_block_affine_scan_fwd(P(A), P(b), P(h0), P(h), B, T, d, k, P(ws), ws.numel(), stream)
    assert rc == 0, rc
    return h, ws


def _noalloc(lib, A, b, h0, B, T, d, k, stream):
    h = torch.full((B, T, d), float("nan"), dtype=torch.float32, device=A.device)
    rc = lib.mgs_block_affine_scan_fwd_noalloc(P(A), P(b), P(h0), P(h), B, T, d, k, stream)
    assert rc == 0, rc
    return h


def test_noalloc_matches_the_workspace_entry_point(gpu):
    import scan_linear_rnns_amd as mgs
    lib = mgs.load()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    cases = [(16, 1024, 64, 8, "zero", 0),     # long-T workload: 8 tiles along T, h0 = NULL
             (2, 300, 16, 8, "normal", 1),     # ragged, smaller: 3 tiles along T, h0 given
             (128, 64, 64, 8, "zero", 2)]      # lab shape: one tile along T
    for rep in range(2):   # the whole sequence twice: the scratch holds words of every shape
        for B, T, d, k, h0k, seed in cases:
            say(f"noalloc B={B} T={T} d={d} k={k} h0={h0k} seed={seed} pass {rep}")
            inp = block_inputs(B, T, d, k=k, seed=seed, h0=h0k, with_dP=False)
            A, b, h0 = (to_dev(x, gpu) for x in (inp.A, inp.b, inp.h0))
            ref, ws = _existing(lib, A, b, h0, B, T, d, k, stream)
            got = _noalloc(lib, A, b, h0, B, T, d, k, stream)
            torch.cuda.synchronize()
            assert mgs.mgs_workspace_check(ws) == 0
            r, g = ref.cpu().numpy(), got.cpu().numpy()
            assert np.all(np.isfinite(g)), (B, T, d)
            assert np.array_equal(r, g), (B, T, d, float(np.max(np.abs(r - g))))
