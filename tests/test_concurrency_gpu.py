"""Scans launched on several streams at once give their single-stream results.

Two scans with multi-tile look-back (the block-affine scan and the log-space
scan, both at the long-T shape B=16 T=1024 d=64) run forward and backward on
two side streams at the same time, while a third stream runs unrelated work
(an fp32 matrix product and device copies) that competes for the same compute
units and memory.  Each launch draws its look-back tags from its own
workspace's epoch counter and waits only on lower-numbered workgroups of its
own launch, so sharing the chip changes timing only: every output must equal
the single-stream result bit for bit, on every repetition, and no look-back
wait may hit its spin limit.
"""
import numpy as np
import pytest

from synthetic import block_inputs, log_inputs
from tests.test_parity_gpu import say, ws_clean

pytestmark = pytest.mark.gpu


def _t(x, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).to(dev)


def test_concurrent_streams_match_single_stream(gpu):
    import torch
    import scan_linear_rnns_amd as mgs
    say("concurrent streams: block-affine + log-space + unrelated work")
    blk = block_inputs(16, 1024, 64, k=8, seed=3, with_dP=False)
    lg = log_inputs(16, 1024, 64, seed=3)
    A, b, dh = (_t(x, gpu) for x in (blk.A, blk.b, blk.dh))
    la, lb, lh0, ldh = (_t(x, gpu) for x in (lg.log_a, lg.log_b, lg.log_h0, lg.dh))

    # single-stream references
    h_ref, ws1 = mgs.mgs_block_affine_scan_fwd(A, b, None)
    g_ref = mgs.mgs_block_affine_scan_bwd(A, b, None, h_ref, dh, ws=ws1)
    hl_ref, ws2 = mgs.mgs_scan_log_fwd(la, lb, lh0)
    gl_ref = mgs.mgs_scan_log_bwd(la, lb, lh0, ldh, ws=ws2, fwd_state_valid=True)
    refs = [x.clone() for x in (h_ref, *g_ref, hl_ref, *gl_ref)]

    # outputs and the unrelated work's buffers, allocated before any side stream runs
    h1 = torch.empty_like(h_ref)
    o1 = tuple(torch.empty_like(x) for x in g_ref)
    h2 = torch.empty_like(hl_ref)
    o2 = tuple(torch.empty_like(x) for x in gl_ref)
    x = torch.randn(2048, 2048, device=gpu)
    y = torch.randn(2048, 2048, device=gpu)
    z = torch.empty(2048, 2048, device=gpu)
    src = torch.randn(1 << 24, device=gpu)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    s1, s2, s3 = torch.cuda.Stream(), torch.cuda.Stream(), torch.cuda.Stream()

    for rep in range(5):
        outs = [h1, *o1, h2, *o2]
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        with torch.cuda.stream(s3):
            for _ in range(4):
                torch.mm(x, y, out=z)
                dst.copy_(src)
        mgs.mgs_block_affine_scan_fwd(A, b, None, h=h1, ws=ws1, stream=s1)
        mgs.mgs_scan_log_fwd(la, lb, lh0, h=h2, ws=ws2, stream=s2)
        mgs.mgs_block_affine_scan_bwd(A, b, None, h1, dh, ws=ws1, out=o1, stream=s1)
        mgs.mgs_scan_log_bwd(la, lb, lh0, ldh, ws=ws2, fwd_state_valid=True, out=o2, stream=s2)
        torch.cuda.synchronize()
        ws_clean(ws1)
        ws_clean(ws2)
        for i, (o, r) in enumerate(zip(outs, refs)):
            assert torch.equal(o, r), (rep, i)
