"""Captured-graph replays give the eager results, replay after replay.

The library is captured into a HIP graph (torch.cuda.CUDAGraph) by the
benchmark.  Look-back tags come from a per-workspace epoch on the device, so
replays of one graph never see each other's published words; this test
replays each graph several times, with unrelated eager work and
synchronisations in between, and compares every replay bitwise with the
eager result.
"""
import ctypes

import numpy as np
import pytest

from synthetic import block_inputs, delta_inputs, linear_inputs, log_inputs, mingru_inputs

pytestmark = pytest.mark.gpu


def _t(x, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).to(dev)


def _replays(fn, outs, n=3):
    """Capture fn() into a graph, replay n times; yield cloned outputs per replay."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    res = []
    for r in range(n):
        for o in outs:
            o.fill_(float("nan"))
        junk = torch.randn(1 << 20, device=outs[0].device)
        junk = (junk * 2).sum()          # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        res.append([o.clone() for o in outs])
    return res


def test_log_scan_graph_replays(gpu):
    import torch
    import scan_linear_rnns_amd as mgs
    print("[graph] log scan B=16 T=1024 d=64", flush=True)
    inp = log_inputs(16, 1024, 64, 21)
    la, lb, lh0, dh = (_t(x, gpu) for x in (inp.log_a, inp.log_b, inp.log_h0, inp.dh))
    h, ws = mgs.mgs_scan_log_fwd(la, lb, lh0)
    ref = [h.clone(), *[x.clone() for x in mgs.mgs_scan_log_bwd(la, lb, lh0, dh, ws=ws, fwd_state_valid=True)]]
    outs = [torch.empty_like(la), torch.empty_like(la), torch.empty_like(la), torch.empty_like(lh0)]

    def step():
        mgs.mgs_scan_log_fwd(la, lb, lh0, h=outs[0], ws=ws)
        mgs.mgs_scan_log_bwd(la, lb, lh0, dh, ws=ws, fwd_state_valid=True, out=tuple(outs[1:]))

    for got in _replays(step, outs):
        for a, b in zip(got, ref):
            assert torch.equal(a, b)
    assert mgs.mgs_workspace_check(ws) == 0


@pytest.mark.parametrize("k", [8, 16, 2])
def test_block_scans_graph_replays(gpu, k):
    import torch
    import scan_linear_rnns_amd as mgs
    print(f"[graph] block scans B=16 T=1024 d=64 k={k}", flush=True)
    inp = block_inputs(16, 1024, 64, k=k, seed=22, h0="normal")
    A, b, h0, dh, dP = (_t(x, gpu) for x in (inp.A, inp.b, inp.h0, inp.dh, inp.dP))
    h, ws = mgs.mgs_block_affine_scan_fwd(A, b, h0, k=k)
    gref = mgs.mgs_block_affine_scan_bwd(A, b, h0, h, dh, k=k, ws=ws)
    P, wsm = mgs.mgs_block_matrix_scan_fwd(A, k=k)
    dAm = mgs.mgs_block_matrix_scan_bwd(A, dP, k=k, ws=wsm, fwd_state_valid=True)
    ref = [h.clone(), *[x.clone() for x in gref], P.clone(), dAm.clone()]
    outs = [torch.empty_like(h), torch.empty_like(A), torch.empty_like(b), torch.empty_like(h0),
            torch.empty_like(A), torch.empty_like(A)]

    def step():
        mgs.mgs_block_affine_scan_fwd(A, b, h0, k=k, h=outs[0], ws=ws)
        mgs.mgs_block_affine_scan_bwd(A, b, h0, outs[0], dh, k=k, ws=ws, out=(outs[1], outs[2], outs[3]))
        mgs.mgs_block_matrix_scan_fwd(A, k=k, P=outs[4], ws=wsm)
        mgs.mgs_block_matrix_scan_bwd(A, dP, k=k, ws=wsm, fwd_state_valid=True, dA=outs[5])

    for got in _replays(step, outs):
        for a, b_ in zip(got, ref):
            assert torch.equal(a, b_)
    assert mgs.mgs_workspace_check(ws) == 0 and mgs.mgs_workspace_check(wsm) == 0


def test_linear_scan_graph_replays(gpu):
    import torch
    import scan_linear_rnns_amd as mgs
    print("[graph] linear scan B=16 T=1024 d=64", flush=True)
    inp = linear_inputs(16, 1024, 64, 23)
    a, b, h0, dh = (_t(x, gpu) for x in (inp.a, inp.b, inp.h0, inp.dh))
    h, ws = mgs.mgs_scan_linear_fwd(a, b, h0)
    ref = [h.clone(), *[x.clone() for x in mgs.mgs_scan_linear_bwd(a, b, h0, dh, ws=ws, fwd_state_valid=True)]]
    outs = [torch.empty_like(a), torch.empty_like(a), torch.empty_like(a), torch.empty_like(h0)]

    def step():
        mgs.mgs_scan_linear_fwd(a, b, h0, h=outs[0], ws=ws)
        mgs.mgs_scan_linear_bwd(a, b, h0, dh, ws=ws, fwd_state_valid=True, out=tuple(outs[1:]))

    for got in _replays(step, outs):
        for x, y in zip(got, ref):
            assert torch.equal(x, y)
    assert mgs.mgs_workspace_check(ws) == 0


def test_mingru_scan_graph_replays(gpu):
    import torch
    import scan_linear_rnns_amd as mgs
    print("[graph] minGRU cell + scan B=16 T=1024 d=64", flush=True)
    inp = mingru_inputs(16, 1024, 64, 24)
    k, x, x0, dh = (_t(v, gpu) for v in (inp.k, inp.x, inp.x0, inp.dh))
    h, ws = mgs.mgs_scan_mingru_fwd(k, x, x0)
    ref = [h.clone(), *[v.clone() for v in mgs.mgs_scan_mingru_bwd(k, x, x0, dh, ws=ws, fwd_state_valid=True)]]
    outs = [torch.empty_like(k), torch.empty_like(k), torch.empty_like(k), torch.empty_like(x0)]

    def step():
        mgs.mgs_scan_mingru_fwd(k, x, x0, h=outs[0], ws=ws)
        mgs.mgs_scan_mingru_bwd(k, x, x0, dh, ws=ws, fwd_state_valid=True, out=tuple(outs[1:]))

    for got in _replays(step, outs):
        for a, b in zip(got, ref):
            assert torch.equal(a, b)
    assert mgs.mgs_workspace_check(ws) == 0


def test_givens_scan_graph_replays(gpu):
    import torch
    import scan_linear_rnns_amd as mgs
    print("[graph] givens scan B=16 T=1024 d=64", flush=True)
    inp = block_inputs(16, 1024, 64, seed=25, h0="normal", with_dP=False, return_angles=True)
    th, s, b, h0, dh = (_t(x, gpu) for x in (inp.theta, inp.s, inp.b, inp.h0, inp.dh))
    h, ws = mgs.mgs_givens_scan_fwd(th, s, b, h0)
    ref = [h.clone(), *[x.clone() for x in mgs.mgs_givens_scan_bwd(th, s, h0, h, dh, ws=ws)]]
    outs = [torch.empty_like(h), torch.empty_like(th), torch.empty_like(s), torch.empty_like(b),
            torch.empty_like(h0)]

    def step():
        mgs.mgs_givens_scan_fwd(th, s, b, h0, h=outs[0], ws=ws)
        mgs.mgs_givens_scan_bwd(th, s, h0, outs[0], dh, ws=ws, out=tuple(outs[1:]))

    for got in _replays(step, outs):
        for x, y in zip(got, ref):
            assert torch.equal(x, y)
    assert mgs.mgs_workspace_check(ws) == 0


def test_delta_graph_replays(gpu):
    import torch
    import scan_linear_rnns_amd as mgs
    print("[graph] delta rule B=16 T=1024 d=64", flush=True)
    inp = delta_inputs(16, 1024, 64, 26, s0="normal")
    q, k, v, beta, S0 = (_t(x, gpu) for x in (inp.q, inp.k, inp.v, inp.beta, inp.S0))
    o, ST, ws = mgs.mgs_delta_fwd(q, k, v, beta, S0)
    ref = [o.clone(), ST.clone()]
    outs = [torch.empty_like(o), torch.empty_like(ST)]

    def step():
        mgs.mgs_delta_fwd(q, k, v, beta, S0, o=outs[0], ST=outs[1], ws=ws)

    for got in _replays(step, outs):
        for x, y in zip(got, ref):
            assert torch.equal(x, y)
