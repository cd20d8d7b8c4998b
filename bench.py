#!/usr/bin/env python
"""Benchmark of the minGRU scan engine on one MI355X.

Metric: forward+backward scan throughput in B*T*d elements per second, and the
fraction of the HBM roofline it reaches.  The headline step is one forward +
backward of the block-affine scan at the long-T shape (B=16, T=1024, d=64,
k = 8, fp32; transitions A_t = sigmoid(s_t) R(theta_t) from the Givens-mesh
generator, materialised; seed 0) -- the largest of the five workloads, at
121.6 MB of compulsory traffic per step.  The same run times every other scan
op at its workload (the "ops" object): the log-space scan at the small, lab and
long-T shapes, the block-affine scan at the lab shape, the block cumulative
product at the long-T shape, and the other ops and block sizes of the library.

Method
  * inputs are synthetic (synthetic/__init__.py), resident in HBM before the
    timed region;
  * each op rotates through M copies of its buffers, M >= 512 MiB / (bytes of
    one set), and every timed replay of K calls continues the rotation where
    the previous replay stopped: a call's buffers were last touched >= 512 MiB
    of other buffers earlier, so no call finds its inputs in L2 or in the
    256 MiB Infinity Cache ("rotated").  When K >= M one graph of K calls
    cycles through M sets (M a divisor of K); when K < M there are M / K
    graphs of K calls over disjoint sets, replayed in turn;
  * launches are captured into HIP graphs (torch.cuda.CUDAGraph) and replayed,
    so host launch overhead is not timed; times come from HIP events on the
    stream the graphs run on; median over the replays;
  * after its timed replays every buffer set's workspace is checked for the
    device-side error flag (a look-back wait that gave up); a flagged op is
    reported invalid and the run exits non-zero;
  * compulsory bytes = every input read once + every output written once
    (workspace excluded); % roofline = bytes / time / 8 TB/s (MI355X HBM3E);
  * cpu_baseline: the fp64 oracle (plain C loops) on the headline workload, on
    one host thread and on several threads over independent chains.

Prints ONE JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import concurrent.futures
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_FP32_TFLOPS = 157.3   # MI355X dense fp32 MFMA
PEAK_GBPS = 8000.0
ROTATE_BYTES = 512 << 20
MAX_SETS = 64              # tiny workloads: at most this many buffer sets

METRIC = "fwd+bwd scan throughput (B*T*d elems/s) and % of HBM roofline, 1 GPU"
HEADLINE = "affine_longT"
# dominant kernel of the headline step (the backward; template arguments
# <k, steps per lane, waves, multi-tile>, as rocprofv3 prints them)
HEADLINE_KERNEL = "baffine_bwd_kernel<8,8,8,true>"
BLOCK_SOURCES = ("block_core.hpp", "block_scan.hip", "device.hpp")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ------------------------------------------------------------------ workloads

def compulsory_bytes(op, B, T, d, k=8):
    N, S = B * T * d, B * d
    if op in ("log", "linear", "mingru"):
        return 12 * N + 4 * S, 20 * N + 8 * S
    if op == "affine":  # h0 = 0 is passed as NULL: not read; dh0 written
        return 4 * N * (k + 2), 4 * N * (2 * k + 3) + 4 * S
    if op == "matrix":
        return 8 * N * k, 12 * N * k
    if op == "delta":  # forward only: q, k, v, beta read, o written (S0 = NULL, final state not requested)
        return 16 * N + 4 * B * T, 0
    if op == "givens":  # angles (k(k-1)/2 per block) and gate instead of A; h0 = NULL
        na = k * (k - 1) // 2
        th, sg = 4 * N * na // k, 4 * N // k
        return th + sg + 8 * N, 2 * (th + sg) + 12 * N + 4 * S
    raise ValueError(op)


def rotation_plan(calls, set_bytes, rotate=True):
    """(buffer sets, graphs) so that K = `calls` calls per replay continue one
    cycle through the sets across replays, the cycle holding >= ROTATE_BYTES."""
    m = min(MAX_SETS, max(1, math.ceil(ROTATE_BYTES / set_bytes))) if rotate else 1
    if calls >= m:
        return next(x for x in range(m, calls + 1) if calls % x == 0), 1
    g = math.ceil(m / calls)
    return g * calls, g


class OpRun:
    """Rotated buffer sets of one op with prebuilt ctypes argument lists."""

    def __init__(self, name, op, B, T, d, dev, calls, k=8, rotate=True):
        import numpy as np
        import torch

        import scan_linear_rnns_amd as mgs
        from synthetic import block_inputs, delta_inputs, linear_inputs, log_inputs, mingru_inputs

        self.name, self.op, self.B, self.T, self.d, self.k = name, op, B, T, d, k
        self.N = B * T * d
        self.calls = calls
        self.lib = mgs.load()
        self.fwd_bytes, self.bwd_bytes = compulsory_bytes(op, B, T, d, k)
        t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev)
        if op == "log":
            inp = log_inputs(B, T, d, 0)
            base = [t(inp.log_a), t(inp.log_b), t(inp.log_h0), t(inp.dh)]
            ws_bytes = mgs.mgs_scan_log_workspace_size(B, T, d)
        elif op == "mingru":
            inp = mingru_inputs(B, T, d, 0)
            base = [t(inp.k), t(inp.x), t(inp.x0), t(inp.dh)]
            ws_bytes = mgs.mgs_scan_mingru_workspace_size(B, T, d)
        elif op == "givens":
            inp = block_inputs(B, T, d, k=8, seed=0, with_dP=False, return_angles=True)
            base = [t(inp.theta), t(inp.s), t(inp.b), t(inp.dh)]
            ws_bytes = mgs.mgs_givens_scan_workspace_size(B, T, d, 8)
        elif op == "delta":
            inp = delta_inputs(B, T, d, 0)
            base = [t(inp.q), t(inp.k), t(inp.v), t(inp.beta)]
            ws_bytes = mgs.mgs_delta_workspace_size(B, T, d)
        elif op == "linear":
            inp = linear_inputs(B, T, d, 0)
            base = [t(inp.a), t(inp.b), t(inp.h0), t(inp.dh)]
            ws_bytes = mgs.mgs_scan_linear_workspace_size(B, T, d)
        elif op == "affine":
            inp = block_inputs(B, T, d, k=k, seed=0, with_dP=False)
            base = [t(inp.A), t(inp.b), t(inp.dh)]
            ws_bytes = mgs.mgs_block_affine_scan_workspace_size(B, T, d, k)
        else:
            inp = block_inputs(B, T, d, k=k, seed=0, with_dP=True)
            base = [t(inp.A), t(inp.dP)]
            ws_bytes = mgs.mgs_block_matrix_scan_workspace_size(B, T, d, k)
        del inp
        self.sets, self.keep, self.ws = [], [], []
        self._add_set(base, ws_bytes, dev, mgs)
        self.set_bytes = sum(x.numel() * 4 for x in self.keep[0][:-1])   # inputs + outputs, not the workspace
        self.M, self.G = rotation_plan(calls, self.set_bytes, rotate)
        for _ in range(self.M - 1):
            self._add_set(base, ws_bytes, dev, mgs)
        torch.cuda.synchronize()

    def _add_set(self, base, ws_bytes, dev, mgs):
        import torch
        P = lambda x: ctypes.c_void_p(x.data_ptr())
        B, T, d, k, op = self.B, self.T, self.d, self.k, self.op
        xs = [x.clone() for x in base]
        ws = mgs.workspace(ws_bytes, dev)
        if op in ("log", "linear", "mingru"):
            la, lb, lh0, dh = xs
            h = torch.empty_like(la)
            dla, dlb, dlh0 = torch.empty_like(la), torch.empty_like(la), torch.empty_like(lh0)
            fa = (P(la), P(lb), P(lh0), P(h), B, T, d, P(ws), ws.numel())
            ba = (P(la), P(lb), P(lh0), P(dh), P(dla), P(dlb), P(dlh0), B, T, d, P(ws), ws.numel(), 1)
            fn_f = getattr(self.lib, f"mgs_scan_{op}_fwd")
            fn_b = getattr(self.lib, f"mgs_scan_{op}_bwd")
            keep = xs + [h, dla, dlb, dlh0, ws]
        elif op == "delta":
            q, kk, v, beta = xs
            o = torch.empty_like(q)
            fa = (P(q), P(kk), P(v), P(beta), None, P(o), None, B, T, d, P(ws), ws.numel())
            ba = None
            fn_f, fn_b = self.lib.mgs_delta_fwd, None
            keep = xs + [o, ws]
        elif op == "givens":
            th, sg, b, dh = xs
            h = torch.empty_like(b)
            dth, dsg, db, dh0 = (torch.empty_like(th), torch.empty_like(sg), torch.empty_like(b),
                                 torch.empty((B, d), device=b.device))
            fa = (P(th), P(sg), P(b), None, P(h), B, T, d, 8, P(ws), ws.numel())
            ba = (P(th), P(sg), None, P(h), P(dh), P(dth), P(dsg), P(db), P(dh0), B, T, d, 8, P(ws), ws.numel())
            fn_f, fn_b = self.lib.mgs_givens_scan_fwd, self.lib.mgs_givens_scan_bwd
            keep = xs + [h, dth, dsg, db, dh0, ws]
        elif op == "affine":
            A, b, dh = xs
            h = torch.empty_like(b)
            dA, db, dh0 = torch.empty_like(A), torch.empty_like(b), torch.empty((B, d), device=b.device)
            fa = (P(A), P(b), None, P(h), B, T, d, k, P(ws), ws.numel())
            ba = (P(A), None, None, P(h), P(dh), P(dA), P(db), P(dh0), B, T, d, k, P(ws), ws.numel())
            fn_f, fn_b = self.lib.mgs_block_affine_scan_fwd, self.lib.mgs_block_affine_scan_bwd
            keep = xs + [h, dA, db, dh0, ws]
        else:
            A, dP = xs
            Pm, dA = torch.empty_like(A), torch.empty_like(A)
            fa = (P(A), P(Pm), B, T, d, k, P(ws), ws.numel())
            ba = (P(A), P(dP), P(dA), B, T, d, k, P(ws), ws.numel(), 1)
            fn_f, fn_b = self.lib.mgs_block_matrix_scan_fwd, self.lib.mgs_block_matrix_scan_bwd
            keep = xs + [Pm, dA, ws]
        self.sets.append((fn_f, fa, fn_b, ba))
        self.keep.append(keep)
        self.ws.append(ws)

    def call(self, i, which, stream):
        fn_f, fa, fn_b, ba = self.sets[i % self.M]
        if which in ("fwd", "pair"):
            rc = fn_f(*fa, stream)
            if rc:
                raise RuntimeError(f"{self.name} fwd status {rc}")
        if which in ("bwd", "pair") and fn_b is not None:
            rc = fn_b(*ba, stream)
            if rc:
                raise RuntimeError(f"{self.name} bwd status {rc}")

    def prime(self):
        """One eager fwd per set so bwd-only graphs have valid forward state."""
        import torch
        s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        for i in range(self.M):
            self.call(i, "fwd", s)
        torch.cuda.synchronize()

    def error_flags(self):
        """OR of the device-side error flags of every set's workspace (clears them)."""
        import torch
        s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        out = 0
        for ws in self.ws:
            f = ctypes.c_int(0)
            rc = self.lib.mgs_workspace_check(ctypes.c_void_p(ws.data_ptr()), s, ctypes.byref(f))
            if rc:
                raise RuntimeError(f"{self.name}: mgs_workspace_check status {rc}")
            out |= f.value
        return out

    def coverage(self):
        return {"buffer_sets": self.M, "graphs": self.G, "calls_per_replay": self.calls,
                "sets_touched_per_replay": min(self.calls, self.M),
                "set_bytes": self.set_bytes, "rotation_bytes": self.M * self.set_bytes}


def graph_time(run: OpRun, which: str, warmup: int, repeats: int = 5):
    """Median over timed replays of (elapsed / calls) in microseconds.  The
    replays continue the buffer rotation: graph g holds calls g*K .. g*K+K-1
    (K = run.calls), and the graphs are replayed in turn."""
    import torch
    K = run.calls
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        s = ctypes.c_void_p(side.cuda_stream)
        for i in range(max(warmup, 1)):
            run.call(i, which, s)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graphs = []
    for gi in range(run.G):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
            for i in range(K):
                run.call(gi * K + i, which, s)
        graphs.append(g)
    for g in graphs:   # one untimed replay of every graph: the rotation is in steady state
        g.replay()
    torch.cuda.synchronize()
    n_rep = run.G * max(1, math.ceil(repeats / run.G))
    times = []
    for r in range(n_rep):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        graphs[r % run.G].replay()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) * 1e3 / K)
    times.sort()
    del graphs
    return times[len(times) // 2]


def stream_time(run: OpRun, which: str, warmup: int):
    """Eager stream launches from Python (includes host launch overhead)."""
    import torch
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for i in range(warmup):
        run.call(i, which, s)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(run.calls):
        run.call(i, which, s)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / run.calls


def copy_bandwidth(dev):
    """Device-to-device copy of 1 GiB: (read + write bytes) / time."""
    import torch
    n = 1 << 28
    a = torch.empty(n, dtype=torch.float32, device=dev).fill_(1.0)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 10
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    sec = e0.elapsed_time(e1) / 1e3 / reps
    del a, b
    return 2 * n * 4 / sec / 1e9


def cold_copy_floor(dev, nbytes, calls, warmup):
    """A device copy moving `nbytes` in total (nbytes/2 read + nbytes/2 written), on
    buffers rotated like the ops' inputs (>= 512 MiB per cycle, the cycle
    continued across replays), captured in graphs: microseconds per copy.  The
    streaming rate this chip reaches for a transfer of this size from cold memory,
    for comparison with a step that moves as much."""
    import torch
    n = max(1, nbytes // 8)   # floats per buffer
    m, G = rotation_plan(calls, 8 * n)
    src = [torch.ones(n, dtype=torch.float32, device=dev) for _ in range(m)]
    dst = [torch.empty(n, dtype=torch.float32, device=dev) for _ in range(m)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(max(warmup, 1)):
            dst[i % m].copy_(src[i % m])
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graphs = []
    for gi in range(G):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(calls):
                j = (gi * calls + i) % m
                dst[j].copy_(src[j])
        graphs.append(g)
    for g in graphs:
        g.replay()
    torch.cuda.synchronize()
    times = []
    for r in range(G * max(1, math.ceil(5 / G))):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        graphs[r % G].replay()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) * 1e3 / calls)
    times.sort()
    del graphs, src, dst
    torch.cuda.empty_cache()
    return times[len(times) // 2]


def cold_copy_reference(dev, nbytes, step_us, calls, warmup, label):
    """One copy of a step's compulsory bytes and two copies of half of them (the
    shape of a forward then a backward launch), against the step's time."""
    one = cold_copy_floor(dev, nbytes, calls, warmup)
    half = cold_copy_floor(dev, nbytes // 2, calls, warmup)
    log(f"cold copy of {label}'s {nbytes / 1e6:.1f} MB: {one:.2f} us ({nbytes / (one * 1e-6) / 1e12:.2f} TB/s); "
        f"two copies of half: {2 * half:.2f} us; the step: {step_us:.2f} us")
    return {"workload": label, "bytes": nbytes, "us_one_copy_of_step_bytes": one,
            "GBps_one_copy": nbytes / (one * 1e-6) / 1e9,
            "us_two_copies_of_half": 2 * half, "step_us": step_us,
            "step_over_two_copies": step_us / (2 * half)}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(seconds):
    """The fp64 oracle (plain C loops, as the tests use it) on the headline
    workload: forward + backward of the block-affine scan, B=16 T=1024 d=64
    k=8.  Half of `seconds` on one thread, half on several threads, each thread
    running the oracle on its own slice of the batch (the chains are independent,
    so the slices' results are exactly the whole batch's)."""
    import numpy as np

    import oracle
    from synthetic import block_inputs
    B, T, d, k = 16, 1024, 64, 8
    inp = block_inputs(B, T, d, k=k, seed=0, with_dP=False)
    A, b, dh = (np.ascontiguousarray(x, dtype=np.float64) for x in (inp.A, inp.b, inp.dh))
    N = B * T * d

    def step(lo, hi):
        oracle.block_affine_fwd(A[lo:hi], b[lo:hi], None, k)
        oracle.block_affine_bwd(A[lo:hi], b[lo:hi], None, dh[lo:hi], k)

    step(0, 1)   # build/load outside the timed region
    n1, t0 = 0, time.perf_counter()
    while True:
        step(0, B)
        n1 += 1
        el1 = time.perf_counter() - t0
        if el1 >= seconds / 2:
            break
    threads = max(1, min(16, B, os.cpu_count() or 1))
    cuts = [B * i // threads for i in range(threads + 1)]
    nt = 0
    with concurrent.futures.ThreadPoolExecutor(max_workers=threads) as pool:
        t0 = time.perf_counter()
        while True:
            list(pool.map(lambda i: step(cuts[i], cuts[i + 1]), range(threads)))
            nt += 1
            elt = time.perf_counter() - t0
            if elt >= seconds / 2:
                break
    v1, vt = n1 * N / el1, nt * N / elt
    return {"value": vt, "unit": "B*T*d elems/s", "cores": threads, "kind": "oracle",
            "value_1_thread": v1, "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "sample": f"block-affine scan fwd+bwd, B=16 T=1024 d=64 k=8 (the headline workload, whole batch), "
                      f"fp64 C loops; {threads} threads each on B/{threads} of the batch: {nt} passes in "
                      f"{elt:.1f} s; one thread: {n1} passes in {el1:.1f} s"}


def kernel_source_hash(names=None):
    """sha256 prefix over the kernel sources (all of csrc, or the named files)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "scan_linear_rnns_amd", "csrc")
    for name in sorted(names if names is not None else os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(kernel_key, profile, sources):
    """HBM bytes per launch from a committed PMC summary, if it was taken on the current sources."""
    path = os.path.join(ROOT, "profiles", profile)
    if not os.path.exists(path):
        return None
    src_hash, value = None, None
    for line in open(path):
        parts = line.split()
        if len(parts) == 2 and parts[0] == "source_hash":
            src_hash = parts[1]
        if len(parts) == 3 and parts[0] == "traffic_bytes_per_launch" and parts[1] == kernel_key:
            value = int(parts[2])
    if src_hash != kernel_source_hash(sources):
        return None
    return value


SPECS = [
    # the five workloads: log space (tiny, lab, long T), block-affine (lab, long T), and the
    # cumulative product at long T; the headline is the block-affine long-T step
    ("affine_longT", "affine", 16, 1024, 64),
    ("log_tiny", "log", 2, 64, 16),
    ("log_lab", "log", 128, 64, 64),
    ("log_longT", "log", 16, 1024, 64),
    ("affine_lab", "affine", 128, 64, 64),
    ("matrix_longT", "matrix", 16, 1024, 64),
    # the other ops of the library
    ("mingru_lab", "mingru", 128, 64, 64),
    ("mingru_longT", "mingru", 16, 1024, 64),
    ("linear_lab", "linear", 128, 64, 64),
    ("linear_longT", "linear", 16, 1024, 64),
    ("givens_lab", "givens", 128, 64, 64),
    ("givens_longT", "givens", 16, 1024, 64),
    # the block ops at the other block sizes of the envelope, long-T shape
    ("affine_k16_longT", "affine", 16, 1024, 64, 16),
    ("matrix_k16_longT", "matrix", 16, 1024, 64, 16),
    ("affine_k4_longT", "affine", 16, 1024, 64, 4),
    ("affine_k1_longT", "affine", 16, 1024, 64, 1),
    # the delta rule's chunked-WY forward
    ("delta_lab", "delta", 128, 64, 64),
    ("delta_longT", "delta", 16, 1024, 64),
]

OP_TEXT = {
    "matrix": "block cumulative product (b = 0), k = {k}",
    "affine": "block-affine scan, k = {k}",
    "givens": "Givens angle-fused block-affine scan (inputs theta, s), k = 8",
    "delta": "delta rule (DeltaNet), chunked-WY forward only (pair = forward), d = 64",
    "linear": "linear-space scan, signed gates",
    "mingru": "minGRU cell fused ahead of the log-space scan (inputs k, x, x0)",
    "log": "log-space scan",
}


def time_op(name, op, B, T, d, k, dev, K, W, warm):
    import torch
    log(f"op {name}: building buffers")
    run = OpRun(name, op, B, T, d, dev, K, k=k)
    run.prime()
    fwd_only = op == "delta"
    pair = graph_time(run, "pair", W)
    fwd = graph_time(run, "fwd", W)
    bwd = None if fwd_only else graph_time(run, "bwd", W)
    eager = stream_time(run, "pair", W)
    flags = run.error_flags()
    tot = run.fwd_bytes + run.bwd_bytes
    rec = {
        "op": OP_TEXT[op].format(k=k),
        "B": B, "T": T, "d": d, "k": k if op in ("affine", "matrix", "givens") else None,
        **run.coverage(),
        "us_per_fwd_bwd": pair, "us_fwd": fwd, "us_bwd": bwd,
        "us_per_fwd_bwd_eager_launch": eager,
        "elems_per_s": run.N / (pair * 1e-6),
        "compulsory_bytes": tot,
        "GBps": tot / (pair * 1e-6) / 1e9,
        "roofline_frac": tot / (pair * 1e-6) / 1e9 / PEAK_GBPS,
        "fwd_roofline_frac": run.fwd_bytes / (fwd * 1e-6) / 1e9 / PEAK_GBPS,
        "bwd_roofline_frac": None if fwd_only else run.bwd_bytes / (bwd * 1e-6) / 1e9 / PEAK_GBPS,
        "workspace_error_flags": flags,
    }
    if flags:
        rec["invalid"] = "a look-back wait hit its spin limit: results of the timed calls are invalid"
    if fwd_only:
        # the recurrence's own work: S k, the rank-1 update and S q, 6 d^2 flops per step
        flops = 6 * d * d * B * T
        rec["algorithmic_flops"] = flops
        rec["TFLOPs"] = flops / (fwd * 1e-6) / 1e12
        rec["mfma_fp32_frac"] = rec["TFLOPs"] / PEAK_FP32_TFLOPS
    if warm:
        # same buffers every call: cache-resident, labelled as such
        warm_run = OpRun(name + "_warm", op, B, T, d, dev, K, k=k, rotate=False)
        warm_run.prime()
        rec["us_per_fwd_bwd_warm_cache_resident"] = graph_time(warm_run, "pair", W)
        del warm_run
    bwd_txt = "-" if bwd is None else f"{bwd:.2f}"
    log(f"op {name}: pair {pair:.2f} us (fwd {fwd:.2f}, bwd {bwd_txt}; eager {eager:.2f}) "
        f"-> {rec['elems_per_s']:.3e} elem/s, {rec['roofline_frac'] * 100:.1f}% of HBM roofline; "
        f"{run.M} sets x {run.set_bytes / 2**20:.1f} MiB, {run.G} graph(s); flags {flags}")
    fb = (run.N, run.fwd_bytes, run.bwd_bytes)
    del run
    torch.cuda.empty_cache()
    return rec, fb


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=40, help="timed calls per replay (K)")
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ops", action="store_true", help="time only the headline step")
    ap.add_argument("--only", default=None, help="comma list of op names to time (profiling runs)")
    ap.add_argument("--warm", action="store_true",
                    help="also time every op on one buffer set (cache-resident figures)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a device copy of exactly 64 MiB (calibrates HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(json.dumps({"error": "one GPU only: the scan's chains are independent, so N GPUs would each "
                                   "run the same kernels on their own B/N shard with no exchange; run with "
                                   "--gpus 1"}), flush=True)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}), flush=True)
        sys.exit(1)
    dev = torch.device("cuda:0")
    K, W = args.steps, args.warmup
    gpu_name = torch.cuda.get_device_name(0)
    log(f"device {gpu_name}; steps={K} warmup={W}")

    only = set(args.only.split(",")) if args.only else None
    if args.copy_calibration:
        # a plain copy of known size: 64 MiB read + 64 MiB written per dispatch
        ca = torch.ones(16 << 20, dtype=torch.float32, device=dev)
        cb = torch.empty_like(ca)
        for _ in range(3):
            cb.copy_(ca)
        torch.cuda.synchronize()
        del ca, cb
    specs = SPECS[:1] if args.no_ops else SPECS
    if only:
        specs = [s for s in specs if s[0] in only]

    ops, sizes = {}, {}
    for name, op, B, T, d, *kk in specs:
        k = kk[0] if kk else 8
        ops[name], sizes[name] = time_op(name, op, B, T, d, k, dev, K, W, args.warm)

    out = {"metric": METRIC, "n_gpus": 1, "steps": K, "warmup": W, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic"}
    head = ops.get(HEADLINE)
    if head is not None:
        N, fwd_b, bwd_b = sizes[HEADLINE]
        pair, bwd = head["us_per_fwd_bwd"], head["us_bwd"]
        out.update({
            "value": N / (pair * 1e-6),
            "unit": "B*T*d elems/s",
            "ms_per_step": pair * 1e-3,
            "hbm_roofline_frac": head["roofline_frac"],
            "config": {"workload": "block-affine scan h_t = A_t h_{t-1} + b_t, forward + backward, long-T shape "
                                   "B=16 T=1024 d=64, k=8 blocks, fp32; A_t = sigmoid(s_t) R(theta_t) from an "
                                   "8-layer Givens mesh (materialised), b and dL/dh ~ N(0,1), h0 = 0, seed 0",
                       "B": 16, "T": 1024, "d": 64, "k": 8,
                       "buffer_sets": head["buffer_sets"], "graphs": head["graphs"],
                       "launch": "hipGraph replay", "gpu": gpu_name},
        })
        achieved = bwd_b / (bwd * 1e-6) / 1e9
        out["roofline"] = {
            "kernel": f"{HEADLINE_KERNEL} (block-affine backward, fused reverse scan, dA formed in registers)",
            "bound": "hbm", "achieved": achieved, "peak": PEAK_GBPS, "unit": "GB/s",
            "frac": achieved / PEAK_GBPS,
            "algorithmic_bytes_per_launch": bwd_b,
            "avg_launch_us": bwd,
            "traffic": traffic_from_profiles("affine_longT_bwd", "block_scans_hbm_traffic.txt", BLOCK_SOURCES),
        }
        if head.get("invalid"):
            out["invalid"] = head["invalid"]
    if not args.no_ops and not only:
        log("copy bandwidth")
        out["copy_GBps"] = copy_bandwidth(dev)
        refs = []
        for name in (HEADLINE, "log_longT"):
            if name in ops:
                r = ops[name]
                refs.append(cold_copy_reference(dev, r["compulsory_bytes"], r["us_per_fwd_bwd"], K, W, name))
        out["cold_copy_reference"] = refs
    out["ops"] = ops
    out["kernel_source_hash"] = kernel_source_hash()
    if not args.no_cpu_baseline and head is not None:
        log(f"cpu baseline (~{args.cpu_seconds:.0f} s)")
        out["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(out), flush=True)
    bad = [n for n, r in ops.items() if r.get("invalid")]
    if bad:
        log(f"invalid ops (workspace error flag set): {bad}")
        sys.exit(3)


if __name__ == "__main__":
    main()
