"""GPU parity of the minGRU cell fused ahead of the log-space scan (mgs_scan_mingru_*).

Every output (h, dk, dx, dx0) element by element against the fp64 oracle
(oracle.mingru_fwd / mingru_bwd) on the same fp32 pre-activations, with the
floored relative rule of tests/test_parity_gpu.py and the log-space scan's bar
of 1e-4 (the cell adds a handful of correctly rounded transcendentals per
element ahead of the same scan).
"""
import numpy as np
import pytest

import oracle
from synthetic import mingru_inputs
from tests.test_parity_gpu import LOG_TOL, floored_err, say, to_dev, to_np, ws_clean

pytestmark = pytest.mark.gpu


def run_mingru(k, x, x0, dh, dev, fwd_state_valid=True):
    import scan_linear_rnns_amd as mgs
    kt, xt, x0t, dht = (to_dev(v, dev) for v in (k, x, x0, dh))
    h, ws = mgs.mgs_scan_mingru_fwd(kt, xt, x0t)
    if fwd_state_valid:
        dk, dx, dx0 = mgs.mgs_scan_mingru_bwd(kt, xt, x0t, dht, ws=ws, fwd_state_valid=True)
    else:
        ws2 = mgs.workspace(ws.numel(), dev)
        dk, dx, dx0 = mgs.mgs_scan_mingru_bwd(kt, xt, x0t, dht, ws=ws2, fwd_state_valid=False)
        ws_clean(ws2)
    ws_clean(ws)
    out = dict(h=to_np(h), dk=to_np(dk), dx=to_np(dx), dx0=to_np(dx0))
    ref = dict(h=oracle.mingru_fwd(k, x, x0))
    ref["dk"], ref["dx"], ref["dx0"] = oracle.mingru_bwd(k, x, x0, dh)
    return out, ref


def check(out, ref):
    for key in out:
        e = floored_err(out[key], ref[key])
        assert e <= LOG_TOL, (key, e)


CASES = [("mingru_tiny", 2, 64, 16), ("mingru_lab", 128, 64, 64), ("mingru_longT", 16, 1024, 64)]


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("name,B,T,d", CASES, ids=[c[0] for c in CASES])
def test_mingru_configs(gpu, name, B, T, d, seed):
    say(f"mingru {name} B={B} T={T} d={d} seed={seed}")
    inp = mingru_inputs(B, T, d, seed)
    check(*run_mingru(inp.k, inp.x, inp.x0, inp.dh, gpu))


@pytest.mark.parametrize("B,T,d", [(1, 1, 8), (3, 65, 16), (2, 129, 32), (2, 1000, 8), (5, 7, 1), (4, 300, 100)])
def test_mingru_edges(gpu, B, T, d):
    say(f"mingru edge B={B} T={T} d={d}")
    inp = mingru_inputs(B, T, d, 5)
    check(*run_mingru(inp.k, inp.x, inp.x0, inp.dh, gpu))


@pytest.mark.parametrize("T", [64, 1024])
def test_mingru_bwd_without_forward_state(gpu, T):
    say(f"mingru bwd recompute-carries T={T}")
    inp = mingru_inputs(4, T, 64, 3)
    check(*run_mingru(inp.k, inp.x, inp.x0, inp.dh, gpu, fwd_state_valid=False))


def test_mingru_saturated_and_kink_inputs(gpu):
    """Saturated gates (|k| up to 40), candidates at g's kink (x = 0 exactly) and deep in
    its sigmoid branch (x down to -40), and the same for x0."""
    say("mingru saturated / kink inputs")
    inp = mingru_inputs(2, 600, 32, 12)
    k, x, x0 = inp.k.copy(), inp.x.copy(), inp.x0.copy()
    k[:, ::5, :8] = 40.0
    k[:, 1::5, :8] = -40.0
    k[:, :, 8:12] *= 12.0
    x[:, ::4, 12:16] = 0.0
    x[:, 2::4, 16:20] = -40.0
    x[:, :, 20:24] *= 10.0
    x0[0, :8] = 0.0
    x0[1, :8] = -30.0
    check(*run_mingru(k, x, x0, inp.dh, gpu))


def test_mingru_determinism(gpu):
    import torch
    import scan_linear_rnns_amd as mgs
    say("mingru determinism")
    inp = mingru_inputs(16, 1024, 64, 13)
    k, x, x0, dh = (to_dev(v, gpu) for v in (inp.k, inp.x, inp.x0, inp.dh))
    first = None
    for _ in range(3):
        h, ws = mgs.mgs_scan_mingru_fwd(k, x, x0)
        g = mgs.mgs_scan_mingru_bwd(k, x, x0, dh, ws=ws, fwd_state_valid=True)
        cur = [h.clone()] + [v.clone() for v in g]
        if first is None:
            first = cur
        else:
            for a, b in zip(first, cur):
                assert torch.equal(a, b)
