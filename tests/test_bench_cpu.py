"""Host-side checks of bench.py: the compulsory-byte counts behind every
roofline fraction, and the one-GPU contract of the command line.

The byte counts are written out here as numbers worked by hand from the shapes
(every input read once, every output written once, workspace excluded), so a
changed formula in bench.py fails against them rather than against itself.
"""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

# (op, B, T, d, k) -> (forward bytes, backward bytes)
CASES = [
    # log space, lab shape: N = 524288, S = 8192.  Forward reads log a, log b
    # (8N) and log h0 (4S), writes h (4N); backward reads log a, log b, dh (12N)
    # and log h0 (4S), writes two gradients (8N) and d log h0 (4S).
    (("log", 128, 64, 64, 8), (6_324_224, 10_551_296)),
    # log space, long T: N = 1048576, S = 1024
    (("log", 16, 1024, 64, 8), (12_587_008, 20_979_712)),
    # the linear scan and the fused minGRU cell move the same tensors
    (("linear", 128, 64, 64, 8), (6_324_224, 10_551_296)),
    (("mingru", 16, 1024, 64, 8), (12_587_008, 20_979_712)),
    # block-affine, k = 8, lab shape, h0 = 0 passed as NULL (not read): forward
    # reads A (64 floats per 8 channels: 8N floats) and b (N), writes h (N):
    # 40N bytes; backward reads A, h, dh (10N floats), writes dA and db (9N
    # floats) and dh0 (S floats): 76N + 4S bytes
    (("affine", 128, 64, 64, 8), (20_971_520, 39_878_656)),
    (("affine", 16, 1024, 64, 8), (41_943_040, 79_695_872)),
    # cumulative product, k = 8, long T: forward reads A, writes P (2 x 8N
    # floats); backward reads A and dP, writes dA (3 x 8N floats)
    (("matrix", 16, 1024, 64, 8), (67_108_864, 100_663_296)),
    # block-affine at k = 16: A is 16N floats
    (("affine", 16, 1024, 64, 16), (75_497_472, 146_804_736)),
    # Givens angle-fused, k = 8, lab shape: 28 angles and one gate per 8
    # channels (3.625N floats) instead of A; forward reads them and b, writes h;
    # backward reads them, h, dh, writes their gradients, db and dh0
    (("givens", 128, 64, 64, 8), (11_796_480, 21_528_576)),
]


@pytest.mark.parametrize("args,expected", CASES)
def test_compulsory_bytes(args, expected):
    op, B, T, d, k = args
    assert bench.compulsory_bytes(op, B, T, d, k) == expected


def test_delta_forward_bytes():
    # q, k, v read (12N), beta read (4BT), o written (4N); forward only
    assert bench.compulsory_bytes("delta", 128, 64, 64) == (8_421_376, 0)


def test_more_than_one_gpu_is_refused():
    """One GPU only: --gpus N > 1 exits with a message and a non-zero status,
    before anything touches a GPU."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    line = r.stdout.strip().splitlines()[-1]
    assert "one GPU only" in json.loads(line)["error"]


@pytest.mark.parametrize("calls", [1, 5, 7, 20, 40, 43, 100, 200])
@pytest.mark.parametrize("set_bytes", [80 << 20, 12 << 20, 33 << 20, 600 << 20, 50_000])
def test_rotation_continues_across_replays(calls, set_bytes):
    """Every timed replay has exactly `calls` calls, and over consecutive replays
    (graph g holds calls g*K .. g*K+K-1, graphs replayed in turn) each buffer set
    is reused only after >= 512 MiB of other sets, unless the set count is capped
    for tiny workloads; every set is touched."""
    M, G = bench.rotation_plan(calls, set_bytes)
    seq = []
    for r in range(3 * G + 2):
        g = r % G
        seq += [(g * calls + i) % M for i in range(calls)]
    assert set(seq) == set(range(M))
    last = {}
    gaps = []
    for pos, s in enumerate(seq):
        if s in last:
            gaps.append(pos - last[s])
        last[s] = pos
    want = min(bench.MAX_SETS, -(-bench.ROTATE_BYTES // set_bytes))
    assert min(gaps) == M >= want
    if M < bench.MAX_SETS:
        assert M * set_bytes >= bench.ROTATE_BYTES


def test_rotation_of_the_headline():
    # block-affine long T: A, b, dh, h, dA, db, dh0 = 80 MiB + 4 KiB per set
    set_bytes = (8 + 1 + 1 + 1 + 8 + 1) * 4 * 16 * 1024 * 64 + 4 * 16 * 64
    assert bench.rotation_plan(20, set_bytes) == (10, 1)
    assert bench.rotation_plan(40, set_bytes) == (8, 1)
    assert bench.rotation_plan(5, set_bytes) == (10, 2)
