#!/usr/bin/env python
"""Benchmark of the minGRU scan engine on one MI355X.

Metric: forward+backward scan throughput in B*T*d elements per second, and the
fraction of the HBM roofline it reaches.  The headline step is one forward +
backward of the log-space minGRU scan at the lab shape (B=128, T=64, d=64,
fp32, MinGRU gate generator, seed 0).  The same run also times every other
scan op at its workload (the "ops" object): the small log case, the long-T log
case, the block-affine scan at the lab and long-T shapes and the block
cumulative product at the long-T shape.

Method
  * inputs are synthetic (synthetic/__init__.py), resident in HBM before the
    timed region;
  * each op cycles through M copies of its buffers whose total is >= 512 MiB,
    so no call finds its inputs in L2 or in the 256 MiB Infinity Cache left by
    an earlier call ("rotated"); a "warm" figure (one buffer set) is reported
    beside it;
  * launches are captured once into a HIP graph (torch.cuda.CUDAGraph) and
    replayed, so host launch overhead is not timed; times come from HIP events
    on the stream the graph runs on;
  * compulsory bytes = every input read once + every output written once
    (workspace excluded); % roofline = bytes / time / 8 TB/s (MI355X HBM3E peak);
  * cpu_baseline: the fp64 oracle (plain C, one thread) on the same headline
    workload, repeated for about --cpu-seconds.

Prints ONE JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
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


class OpRun:
    """M rotated buffer sets of one op with prebuilt ctypes argument lists."""

    def __init__(self, name, op, B, T, d, dev, rotate=True, k=8):
        import numpy as np
        import torch

        import scan_linear_rnns_amd as mgs
        from synthetic import block_inputs, delta_inputs, linear_inputs, log_inputs, mingru_inputs

        self.name, self.op, self.B, self.T, self.d, self.k = name, op, B, T, d, k
        self.N = B * T * d
        self.lib = mgs.load()
        self.fwd_bytes, self.bwd_bytes = compulsory_bytes(op, B, T, d, k)
        t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev)
        P = lambda x: ctypes.c_void_p(x.data_ptr())
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
        else:
            inp = block_inputs(B, T, d, k=k, seed=0, with_dP=(op == "matrix"))
            base = [t(inp.A), t(inp.b), t(inp.dh)] + ([t(inp.dP)] if op == "matrix" else [])
            sz = mgs.mgs_block_affine_scan_workspace_size if op == "affine" else mgs.mgs_block_matrix_scan_workspace_size
            ws_bytes = sz(B, T, d, k)
        per_set = sum(x.numel() * 4 for x in base) * 2
        self.M = max(1, math.ceil(ROTATE_BYTES / per_set)) if rotate else 1
        self.sets = []
        self.keep = []
        for _ in range(self.M):
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
                                     torch.empty((B, d), device=dev))
                fa = (P(th), P(sg), P(b), None, P(h), B, T, d, 8, P(ws), ws.numel())
                ba = (P(th), P(sg), None, P(h), P(dh), P(dth), P(dsg), P(db), P(dh0), B, T, d, 8, P(ws), ws.numel())
                fn_f, fn_b = self.lib.mgs_givens_scan_fwd, self.lib.mgs_givens_scan_bwd
                keep = xs + [h, dth, dsg, db, dh0, ws]
            elif op == "affine":
                A, b, dh = xs
                h = torch.empty_like(b)
                dA, db, dh0 = torch.empty_like(A), torch.empty_like(b), torch.empty((B, d), device=dev)
                fa = (P(A), P(b), None, P(h), B, T, d, k, P(ws), ws.numel())
                ba = (P(A), None, None, P(h), P(dh), P(dA), P(db), P(dh0), B, T, d, k, P(ws), ws.numel())
                fn_f, fn_b = self.lib.mgs_block_affine_scan_fwd, self.lib.mgs_block_affine_scan_bwd
                keep = xs + [h, dA, db, dh0, ws]
            else:
                A, b, dh, dP = xs
                Pm, dA = torch.empty_like(A), torch.empty_like(A)
                fa = (P(A), P(Pm), B, T, d, k, P(ws), ws.numel())
                ba = (P(A), P(dP), P(dA), B, T, d, k, P(ws), ws.numel(), 1)
                fn_f, fn_b = self.lib.mgs_block_matrix_scan_fwd, self.lib.mgs_block_matrix_scan_bwd
                keep = xs + [Pm, dA, ws]
            self.sets.append((fn_f, fa, fn_b, ba))
            self.keep.append(keep)
        torch.cuda.synchronize()

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


def graph_time(run: OpRun, which: str, steps: int, warmup: int, repeats: int = 5):
    """Median over `repeats` of (elapsed / steps) in microseconds for a graph of
    `steps` consecutive calls (cycling the buffer sets), after `warmup` calls."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        s = ctypes.c_void_p(side.cuda_stream)
        for i in range(max(warmup, 1)):
            run.call(i, which, s)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        for i in range(steps):
            run.call(i, which, s)
    g.replay()      # warm replay
    torch.cuda.synchronize()
    times = []
    for _ in range(repeats):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) * 1e3 / steps)
    times.sort()
    del g
    return times[len(times) // 2]


def stream_time(run: OpRun, which: str, steps: int, warmup: int):
    """Eager stream launches from Python (includes host launch overhead)."""
    import torch
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for i in range(warmup):
        run.call(i, which, s)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        run.call(i, which, s)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / steps


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


def cold_copy_floor(dev, nbytes, steps, warmup):
    """A device copy moving `nbytes` in total (nbytes/2 read + nbytes/2 written), on
    buffers rotated through >= 512 MiB like the ops' inputs, captured in a graph:
    microseconds per copy.  The streaming rate this chip reaches for a transfer of
    this size from cold memory, for comparison with a step that moves as much."""
    import torch
    n = max(1, nbytes // 8)   # floats per buffer
    m = max(1, math.ceil(ROTATE_BYTES / (8 * n)))
    src = [torch.ones(n, dtype=torch.float32, device=dev) for _ in range(m)]
    dst = [torch.empty(n, dtype=torch.float32, device=dev) for _ in range(m)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(max(warmup, 1)):
            dst[i % m].copy_(src[i % m])
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(steps):
            dst[i % m].copy_(src[i % m])
    g.replay()
    torch.cuda.synchronize()
    times = []
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) * 1e3 / steps)
    times.sort()
    del g, src, dst
    torch.cuda.empty_cache()
    return times[len(times) // 2]


def cpu_baseline(seconds):
    import numpy as np

    import oracle
    from synthetic import log_inputs
    inp = log_inputs(128, 64, 64, 0)
    la, lb, lh0, dh = (x.astype(np.float64) for x in (inp.log_a, inp.log_b, inp.log_h0, inp.dh))
    oracle.log_fwd(la[:1], lb[:1], lh0[:1])   # build/load outside the timed region
    n = 0
    t0 = time.perf_counter()
    while True:
        oracle.log_fwd(la, lb, lh0)
        oracle.log_bwd(la, lb, lh0, dh)
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    N = la.size
    return {"value": n * N / el, "unit": "B*T*d elems/s", "cores": 1, "kind": "oracle",
            "sample": f"log-space scan fwd+bwd, B=128 T=64 d=64 (the headline workload), fp64 C loops on one "
                      f"host thread, repeated {n} times over {el:.1f} s"}


LOG_SOURCES = ("elem_scan.hip", "device.hpp")


def kernel_source_hash(names=None):
    """sha256 prefix over the kernel sources (all of csrc, or the named files)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "scan_linear_rnns_amd", "csrc")
    for name in sorted(names if names is not None else os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(kernel_key, profile="elem_scans_lab_hbm_traffic.txt", sources=LOG_SOURCES):
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


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ops", action="store_true", help="time only the headline step")
    ap.add_argument("--only", default=None, help="comma list of op names to time (profiling runs)")
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
    specs = [
        ("log_lab", "log", 128, 64, 64),
        ("log_tiny", "log", 2, 64, 16),
        ("log_longT", "log", 16, 1024, 64),
        ("mingru_lab", "mingru", 128, 64, 64),
        ("mingru_longT", "mingru", 16, 1024, 64),
        ("linear_lab", "linear", 128, 64, 64),
        ("linear_longT", "linear", 16, 1024, 64),
        ("affine_lab", "affine", 128, 64, 64),
        ("affine_longT", "affine", 16, 1024, 64),
        ("givens_lab", "givens", 128, 64, 64),
        ("givens_longT", "givens", 16, 1024, 64),
        ("matrix_longT", "matrix", 16, 1024, 64),
        # the block ops at the other block sizes of the envelope, long-T shape
        ("affine_k16_longT", "affine", 16, 1024, 64, 16),
        ("matrix_k16_longT", "matrix", 16, 1024, 64, 16),
        ("affine_k4_longT", "affine", 16, 1024, 64, 4),
        ("affine_k1_longT", "affine", 16, 1024, 64, 1),
        # the delta rule's chunked-WY forward
        ("delta_lab", "delta", 128, 64, 64),
        ("delta_longT", "delta", 16, 1024, 64),
    ]
    if args.no_ops:
        specs = specs[:1]
    if only:
        specs = [s for s in specs if s[0] in only]

    ops = {}
    head = None
    for name, op, B, T, d, *kk in specs:
        k = kk[0] if kk else 8
        log(f"op {name}: building buffers")
        run = OpRun(name, op, B, T, d, dev, k=k)
        run.prime()
        steps = K if name == "log_lab" else max(20, K // 2)
        fwd_only = op == "delta"
        pair = graph_time(run, "pair", steps, W)
        fwd = graph_time(run, "fwd", steps, W)
        bwd = None if fwd_only else graph_time(run, "bwd", steps, W)
        eager = stream_time(run, "pair", steps, W)
        warm_run = OpRun(name + "_warm", op, B, T, d, dev, rotate=False, k=k)
        warm_run.prime()
        warm = graph_time(warm_run, "pair", steps, W)
        del warm_run
        tot = run.fwd_bytes + run.bwd_bytes
        rec = {
            "B": B, "T": T, "d": d, "k": k if op in ("affine", "matrix", "givens") else None,
            "buffer_sets": run.M, "steps": steps,
            "us_per_fwd_bwd": pair, "us_fwd": fwd, "us_bwd": bwd,
            "us_per_fwd_bwd_eager_launch": eager, "us_per_fwd_bwd_warm": warm,
            "elems_per_s": run.N / (pair * 1e-6),
            "compulsory_bytes": tot,
            "GBps": tot / (pair * 1e-6) / 1e9,
            "roofline_frac": tot / (pair * 1e-6) / 1e9 / PEAK_GBPS,
            "fwd_roofline_frac": run.fwd_bytes / (fwd * 1e-6) / 1e9 / PEAK_GBPS,
            "bwd_roofline_frac": None if fwd_only else run.bwd_bytes / (bwd * 1e-6) / 1e9 / PEAK_GBPS,
        }
        if fwd_only:
            # the recurrence's own work: S k, the rank-1 update and S q, 6 d^2 flops per step
            flops = 6 * d * d * B * T
            rec["algorithmic_flops"] = flops
            rec["TFLOPs"] = flops / (fwd * 1e-6) / 1e12
            rec["mfma_fp32_frac"] = rec["TFLOPs"] / PEAK_FP32_TFLOPS
        if op == "matrix":
            rec["op"] = f"block cumulative product (b = 0), k = {k}"
        elif op == "affine":
            rec["op"] = f"block-affine scan, k = {k}"
        elif op == "givens":
            rec["op"] = "Givens angle-fused block-affine scan (inputs theta, s), k = 8"
        elif op == "delta":
            rec["op"] = "delta rule (DeltaNet), chunked-WY forward only (pair = forward), d = 64"
        elif op == "linear":
            rec["op"] = "linear-space scan, signed gates"
        elif op == "mingru":
            rec["op"] = "minGRU cell fused ahead of the log-space scan (inputs k, x, x0)"
        else:
            rec["op"] = "log-space scan"
        ops[name] = rec
        bwd_txt = "-" if bwd is None else f"{bwd:.2f}"
        log(f"op {name}: pair {pair:.2f} us (fwd {fwd:.2f}, bwd {bwd_txt}; eager {eager:.2f}; warm {warm:.2f}) "
            f"-> {rec['elems_per_s']:.3e} elem/s, {rec['roofline_frac']*100:.1f}% of HBM roofline")
        if name == "log_lab":
            head = (run, pair, bwd)
        else:
            del run
        torch.cuda.empty_cache()

    out = {"metric": "fwd+bwd scan throughput (B*T*d elems/s) and % of HBM roofline, 1 GPU",
           "n_gpus": 1, "steps": K, "warmup": W, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "f32", "data": "synthetic"}
    if head is not None:
        run, pair, bwd = head
        out.update({
            "value": run.N / (pair * 1e-6),
            "unit": "B*T*d elems/s",
            "ms_per_step": pair * 1e-3,
            "hbm_roofline_frac": (run.fwd_bytes + run.bwd_bytes) / (pair * 1e-6) / 1e9 / PEAK_GBPS,
            "config": {"workload": "log-space minGRU scan, forward + backward, lab shape B=128 T=64 d=64 fp32 "
                                   "(MinGRU gate generator, seed 0)",
                       "B": 128, "T": 64, "d": 64, "buffer_sets": run.M, "launch": "hipGraph replay",
                       "gpu": gpu_name},
        })
        achieved = run.bwd_bytes / (bwd * 1e-6) / 1e9
        out["roofline"] = {
            "kernel": "log_bwd_kernel (log-space scan backward, fused forward recompute), lab shape",
            "bound": "hbm", "achieved": achieved, "peak": PEAK_GBPS, "unit": "GB/s",
            "frac": achieved / PEAK_GBPS,
            "algorithmic_bytes_per_launch": run.bwd_bytes,
            "avg_launch_us": bwd,
            "traffic": traffic_from_profiles("log_bwd_lab"),
        }
    if not args.no_ops and not only:
        log("copy bandwidth")
        out["copy_GBps"] = copy_bandwidth(dev)
        if head is not None:
            # the chip's cold streaming rate at the headline step's size: one copy
            # moving the step's compulsory bytes (two of them stand for the step's two
            # dependent launches, each moving about half)
            run = head[0]
            tot = run.fwd_bytes + run.bwd_bytes
            one = cold_copy_floor(dev, tot, max(20, K // 2), W)
            half = cold_copy_floor(dev, tot // 2, max(20, K // 2), W)
            out["cold_copy_reference"] = {
                "bytes": tot, "us_one_copy_of_step_bytes": one,
                "GBps_one_copy": tot / (one * 1e-6) / 1e9,
                "us_two_copies_of_half": 2 * half,
                "step_us": head[1],
                "step_over_two_copies": head[1] / (2 * half),
            }
            log(f"cold copy of the step's {tot / 1e6:.1f} MB: {one:.2f} us ({tot / (one * 1e-6) / 1e12:.2f} TB/s); "
                f"two copies of half: {2 * half:.2f} us; the step: {head[1]:.2f} us")
    out["ops"] = ops
    out["kernel_source_hash"] = kernel_source_hash()
    if not args.no_cpu_baseline and head is not None:
        log(f"cpu baseline (~{args.cpu_seconds:.0f} s)")
        out["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
