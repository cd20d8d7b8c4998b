"""Both publish scopes of the look-back against the oracle.

Tiles publish their look-back words with workgroup-scope stores when every
reader runs on the writer's XCD -- the launch's tiles of one chain group lie
nCG apart in blockIdx and nCG is a multiple of the device's XCD count (8 on an
MI355X in its single-partition mode) -- and with agent-scope stores
otherwise.  Each case below runs several tiles along T at a chain-group
count of each kind:
  log-space scan (64 chains per group, 128 steps per tile): S = B*d = 512
  (nCG = 8) and 448 (nCG = 7), T = 600 (5 tiles);
  block-affine scan and cumulative product at k = 8 (4 chains per group, 128
  steps per tile): B*d/8 = 32 chains (nCG = 8) and 24 (nCG = 6), T = 1000
  (8 tiles).
Every output is held to the parity bars and the workspace's error word must
stay clear (no wait ran to its limit).
"""
import pytest

from tests.test_parity_gpu import BLOCK_TOL, LOG_TOL, floored_err, run_block, run_log, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("B,d,ncg", [(8, 64, 8), (7, 64, 7)])
def test_log_scan_publish_scopes(gpu, B, d, ncg):
    say(f"look-back scope: log B={B} T=600 d={d} (nCG={ncg})")
    out, ref = run_log(B, 600, d, 11, gpu)
    for key in out:
        assert floored_err(out[key], ref[key]) <= LOG_TOL, key


@pytest.mark.parametrize("B,d,ncg", [(4, 64, 8), (3, 64, 6)])
def test_block_scans_publish_scopes(gpu, B, d, ncg):
    say(f"look-back scope: block k=8 B={B} T=1000 d={d} (nCG={ncg})")
    out, ref = run_block(B, 1000, d, 12, gpu)
    for key in out:
        assert floored_err(out[key], ref[key]) <= BLOCK_TOL, key
