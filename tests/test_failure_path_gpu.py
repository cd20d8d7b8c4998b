"""The look-back's failure path, forced from the host.

Every cross-workgroup wait is bounded: after its spin limit it gives up,
raises bit 0 of the workspace's error word and lets its kernel finish.  Here
mgs_workspace_set_waits gives the waits a limit of a few polls and makes each
of them expect a launch tag that no launch publishes, so every wait of a
multi-tile launch gives up -- and every kernel still exits.  The test checks
that mgs_workspace_check reports the flag after the forward and after the
backward, then restores normal operation on the same workspace and checks
that the next forward and backward equal a reference run bit for bit and
leave the flag clear.  Covered: the log-space scan (one look-back lane per
chain), the block-affine scan at k = 8 (half-wave polling units) and k = 16
(whole-wave units), and the cumulative product at k = 8 (whole-wave units
with matrix carries), all at B=16, T=1024 (8 tiles along T).
"""
import numpy as np
import pytest

from synthetic import block_inputs, log_inputs
from tests.test_parity_gpu import say

pytestmark = pytest.mark.gpu

B, T, d = 16, 1024, 64


def _t(x, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).to(dev)


def _fails_then_recovers(run, ws, ref):
    """run(ws, stage) for stage 'fwd' / 'bwd' returns the outputs of that stage."""
    import torch
    import scan_linear_rnns_amd as mgs
    mgs.mgs_workspace_set_waits(ws, spin_limit=4, fail_waits=True)
    run(ws, "fwd")
    torch.cuda.synchronize()
    assert mgs.mgs_workspace_check(ws) & 1, "a forward whose waits cannot succeed raised no flag"
    run(ws, "bwd")
    torch.cuda.synchronize()
    assert mgs.mgs_workspace_check(ws) & 1, "a backward whose waits cannot succeed raised no flag"
    mgs.mgs_workspace_set_waits(ws, 0, False)
    got = run(ws, "fwd") + run(ws, "bwd")
    torch.cuda.synchronize()
    assert mgs.mgs_workspace_check(ws) == 0
    for i, (g, r) in enumerate(zip(got, ref)):
        assert torch.equal(g, r), i


def test_log_scan_waits_give_up_and_recover(gpu):
    import scan_linear_rnns_amd as mgs
    say("failure path: log-space scan")
    x = log_inputs(B, T, d, seed=4)
    la, lb, lh0, dh = (_t(v, gpu) for v in (x.log_a, x.log_b, x.log_h0, x.dh))

    def run(ws, stage):
        if stage == "fwd":
            return (mgs.mgs_scan_log_fwd(la, lb, lh0, ws=ws)[0],)
        return tuple(mgs.mgs_scan_log_bwd(la, lb, lh0, dh, ws=ws, fwd_state_valid=True))

    ws0 = mgs.workspace(mgs.mgs_scan_log_workspace_size(B, T, d), gpu)
    ref = [v.clone() for v in run(ws0, "fwd") + run(ws0, "bwd")]
    assert mgs.mgs_workspace_check(ws0) == 0
    _fails_then_recovers(run, mgs.workspace(ws0.numel(), gpu), ref)


@pytest.mark.parametrize("k", [8, 16])
def test_block_affine_waits_give_up_and_recover(gpu, k):
    import scan_linear_rnns_amd as mgs
    say(f"failure path: block-affine scan k={k}")
    x = block_inputs(B, T, d, k=k, seed=4, with_dP=False)
    A, b, dh = (_t(v, gpu) for v in (x.A, x.b, x.dh))
    h_keep = {}

    def run(ws, stage):
        if stage == "fwd":
            h_keep["h"] = mgs.mgs_block_affine_scan_fwd(A, b, None, k=k, ws=ws)[0]
            return (h_keep["h"],)
        return tuple(mgs.mgs_block_affine_scan_bwd(A, b, None, h_keep["h"], dh, k=k, ws=ws))

    ws0 = mgs.workspace(mgs.mgs_block_affine_scan_workspace_size(B, T, d, k), gpu)
    ref = [v.clone() for v in run(ws0, "fwd") + run(ws0, "bwd")]
    assert mgs.mgs_workspace_check(ws0) == 0
    _fails_then_recovers(run, mgs.workspace(ws0.numel(), gpu), ref)


def test_block_cumprod_waits_give_up_and_recover(gpu):
    import scan_linear_rnns_amd as mgs
    say("failure path: block cumulative product k=8")
    x = block_inputs(B, T, d, k=8, seed=4)
    A, dP = _t(x.A, gpu), _t(x.dP, gpu)

    def run(ws, stage):
        if stage == "fwd":
            return (mgs.mgs_block_matrix_scan_fwd(A, k=8, ws=ws)[0],)
        return (mgs.mgs_block_matrix_scan_bwd(A, dP, k=8, ws=ws, fwd_state_valid=True),)

    ws0 = mgs.workspace(mgs.mgs_block_matrix_scan_workspace_size(B, T, d, 8), gpu)
    ref = [v.clone() for v in run(ws0, "fwd") + run(ws0, "bwd")]
    assert mgs.mgs_workspace_check(ws0) == 0
    _fails_then_recovers(run, mgs.workspace(ws0.numel(), gpu), ref)
