"""GPU parity of the delta rule's chunked-WY forward (mgs_delta_fwd) against the
fp64 oracle (the sequential loop S_t = S_{t-1} + beta_t (v_t - S_{t-1} k_t) k_t^T,
o_t = S_t q_t).

Bars.  The pages fix no tolerance for this op.  Each output is a 64-term dot
product whose terms cancel, so near-zero outputs carry absolute rounding of the
row's scale: on these inputs a plain fp32 sequential loop scores up to 1.8e-4
and an fp32 evaluation of the chunked WY form up to 2.4e-4 under the floored
relative rule, 3e-7 and 4.4e-7 normwise.  The bars are 1e-3 (floored) and 5e-6
(normwise, max |x - r| / max |r|), both per output tensor.
"""
import numpy as np
import pytest

import oracle
from synthetic import delta_inputs
from tests.test_parity_gpu import floored_err, say, to_dev, to_np

pytestmark = pytest.mark.gpu

FLOORED_TOL = 1e-3
NORM_TOL = 5e-6


def normwise(x, r):
    x, r = np.asarray(x, np.float64), np.asarray(r, np.float64)
    if not np.all(np.isfinite(x)):
        return float("inf")
    return float(np.max(np.abs(x - r)) / max(np.max(np.abs(r)), 1e-30))


def run_delta(inp, dev):
    import scan_linear_rnns_amd as mgs
    q, k, v, beta, S0 = (to_dev(x, dev) for x in (inp.q, inp.k, inp.v, inp.beta, inp.S0))
    o, ST, _ = mgs.mgs_delta_fwd(q, k, v, beta, S0)
    ro, rST = oracle.delta_fwd(inp.q, inp.k, inp.v, inp.beta, inp.S0)
    return dict(o=to_np(o), ST=to_np(ST)), dict(o=ro, ST=rST)


def check(out, ref):
    for key in out:
        assert floored_err(out[key], ref[key]) <= FLOORED_TOL, (key, floored_err(out[key], ref[key]))
        assert normwise(out[key], ref[key]) <= NORM_TOL, (key, normwise(out[key], ref[key]))


CASES = [("delta_lab", 128, 64, 64), ("delta_longT", 16, 1024, 64)]


@pytest.mark.parametrize("seed", [0, 1])
@pytest.mark.parametrize("name,B,T,d", CASES, ids=[c[0] for c in CASES])
def test_delta_configs(gpu, name, B, T, d, seed):
    say(f"delta {name} B={B} T={T} seed={seed}")
    out, ref = run_delta(delta_inputs(B, T, d, seed), gpu)
    check(out, ref)


@pytest.mark.parametrize("T", [256, 512, 960, 1024, 1025, 1088])
def test_delta_state_pass_chunk_counts(gpu, T):
    """Sequences of 4, 8, 15 and 16 chunks take the state pass unrolled for
    their chunk count; 17 chunks (T = 1025, a one-step last chunk, and 1088)
    take the looped pass."""
    say(f"delta state pass B=2 T={T} ({(T + 63) // 64} chunks)")
    out, ref = run_delta(delta_inputs(2, T, 64, 9, s0="normal"), gpu)
    check(out, ref)


@pytest.mark.parametrize("B,T", [(1, 1), (3, 7), (2, 63), (2, 64), (2, 65), (1, 129), (3, 300), (1, 2048)])
def test_delta_edges(gpu, B, T):
    say(f"delta edge B={B} T={T} (S0 drawn)")
    out, ref = run_delta(delta_inputs(B, T, 64, 5, s0="normal"), gpu)
    check(out, ref)


def test_delta_beta_zero_keeps_state(gpu):
    import scan_linear_rnns_amd as mgs
    say("delta beta = 0")
    inp = delta_inputs(2, 130, 64, 6, s0="normal")
    q, k, v, S0 = (to_dev(x, gpu) for x in (inp.q, inp.k, inp.v, inp.S0))
    beta = to_dev(np.zeros_like(inp.beta), gpu)
    o, ST, _ = mgs.mgs_delta_fwd(q, k, v, beta, S0)
    assert np.array_equal(to_np(ST), inp.S0)
    want = np.einsum("brc,btc->btr", inp.S0.astype(np.float64), inp.q.astype(np.float64))
    assert normwise(to_np(o), want) <= 1e-6


def test_delta_unit_key_full_write(gpu):
    """beta = 1 with a unit key writes v exactly: S_1 k_1 = v_1 for any S0."""
    import scan_linear_rnns_amd as mgs
    say("delta exact write")
    inp = delta_inputs(4, 1, 64, 7, s0="normal")
    q, k, v, S0 = (to_dev(x, gpu) for x in (inp.q, inp.k, inp.v, inp.S0))
    beta = to_dev(np.ones_like(inp.beta), gpu)
    _, ST, _ = mgs.mgs_delta_fwd(q, k, v, beta, S0)
    got = np.einsum("brc,bc->br", to_np(ST).astype(np.float64), inp.k[:, 0].astype(np.float64))
    assert np.max(np.abs(got - inp.v[:, 0])) <= 1e-4 * np.max(np.abs(inp.S0))


def test_delta_sequence_continuation(gpu):
    """Running T1 steps, then T2 steps from the returned state, equals one run."""
    import scan_linear_rnns_amd as mgs
    say("delta continuation")
    inp = delta_inputs(3, 200, 64, 8, s0="normal")
    q, k, v, beta, S0 = (to_dev(x, gpu) for x in (inp.q, inp.k, inp.v, inp.beta, inp.S0))
    o, ST, _ = mgs.mgs_delta_fwd(q, k, v, beta, S0)
    cut = lambda x, a, b: x[:, a:b].contiguous()
    o1, S1, _ = mgs.mgs_delta_fwd(cut(q, 0, 77), cut(k, 0, 77), cut(v, 0, 77), cut(beta, 0, 77), S0)
    o2, S2, _ = mgs.mgs_delta_fwd(cut(q, 77, 200), cut(k, 77, 200), cut(v, 77, 200), cut(beta, 77, 200), S1)
    # the two runs chunk the steps differently, so they agree to rounding only
    assert normwise(np.concatenate([to_np(o1), to_np(o2)], axis=1), to_np(o)) <= NORM_TOL
    assert normwise(to_np(S2), to_np(ST)) <= NORM_TOL


def test_delta_empty_sequence_passes_state(gpu):
    import torch
    import scan_linear_rnns_amd as mgs
    say("delta T = 0")
    S0 = torch.randn(3, 64, 64, device=gpu)
    e = torch.empty(3, 0, 64, device=gpu)
    _, ST, _ = mgs.mgs_delta_fwd(e, e.clone(), e.clone(), torch.empty(3, 0, device=gpu), S0)
    assert torch.equal(ST, S0)
    _, ST0, _ = mgs.mgs_delta_fwd(e, e.clone(), e.clone(), torch.empty(3, 0, device=gpu), None)
    assert torch.count_nonzero(ST0) == 0


def test_delta_determinism(gpu):
    import torch
    import scan_linear_rnns_amd as mgs
    say("delta determinism")
    inp = delta_inputs(16, 1024, 64, 9)
    q, k, v, beta = (to_dev(x, gpu) for x in (inp.q, inp.k, inp.v, inp.beta))
    first = None
    for _ in range(3):
        o, ST, _ = mgs.mgs_delta_fwd(q, k, v, beta)
        if first is None:
            first = (o.clone(), ST.clone())
        else:
            assert torch.equal(first[0], o) and torch.equal(first[1], ST)


@pytest.mark.parametrize("B,T", [(3, 1), (2, 37), (128, 64)])
def test_delta_single_chunk_from_zero(gpu, B, T):
    """Sequences of one chunk entered from S = 0 take a one-kernel path (the
    state pass reduces to O = M U, S_T = U^T K): against the oracle, and against
    the two-kernel path taken when the same zero state is passed explicitly."""
    import torch
    import scan_linear_rnns_amd as mgs
    say(f"delta single chunk from zero B={B} T={T}")
    inp = delta_inputs(B, T, 64, 12)
    q, k, v, beta = (to_dev(x, gpu) for x in (inp.q, inp.k, inp.v, inp.beta))
    o1, S1, _ = mgs.mgs_delta_fwd(q, k, v, beta, None)
    o2, S2, _ = mgs.mgs_delta_fwd(q, k, v, beta, torch.zeros(B, 64, 64, device=gpu))
    ro, rS = oracle.delta_fwd(inp.q, inp.k, inp.v, inp.beta, None)
    check(dict(o=to_np(o1), ST=to_np(S1)), dict(o=ro, ST=rS))
    assert normwise(to_np(o1), to_np(o2)) <= 1e-6 and normwise(to_np(S1), to_np(S2)) <= 1e-6
    o3, S3, _ = mgs.mgs_delta_fwd(q, k, v, beta, None, want_state=False)
    assert S3 is None and torch.equal(o3, o1)
