"""Builds libmgs.so (the C-ABI scan library) in-tree with hipcc for gfx950.

Usage: python -m scan_linear_rnns_amd.build   (or call build()).
The shared library lands next to this file, where the Python binding loads it.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libmgs.so")
OBJ_DIR = os.path.join(HERE, "_build")   # object files of the last build (the sanitizer test links against them)
# (source, object name, extra flags): block_scan_k.hip is built once per block
# size it serves, each object holding that size's kernels only.
SOURCES = [("mgs_api.cpp", "mgs_api", ()),
           ("elem_scan.hip", "elem_scan", ()),
           ("block_scan.hip", "block_scan", ()),
           ("delta_scan.hip", "delta_scan", ())] + [
          ("block_scan_k.hip", f"block_scan_k{k}", (f"-DMGS_ROWS_K={k}",)) for k in (1, 2, 4, 16)]
JOBS = int(os.environ.get("MGS_BUILD_JOBS", "8"))
ARCH = os.environ.get("MGS_OFFLOAD_ARCH", "gfx950")

# Packed fp32 instructions are disabled for every device code object: the
# compiler would otherwise form them from ordinary float code.
# No packed fp32 instructions anywhere.  No atomic optimizer: it turns the
# one-lane launch-epoch atomic each multi-tile kernel issues at its start into a
# wave-reduced form whose readfirstlane waits for the atomic's round trip
# before the wave's loads go out (and the workgroup then waits for that wave at
# its first barrier).
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-mllvm", "-amdgpu-atomic-optimizer-strategy=None"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the MI355X library cannot be built")


def compile_cmd(src: str, obj: str, extra=()) -> list:
    return [hipcc(), "-x", "hip", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
            "-I", INCLUDE, "-I", CSRC, *DEVICE_FLAGS, *extra, "-c", src, "-o", obj]


def _compile(src: str, obj: str, extra=()) -> None:
    subprocess.run(compile_cmd(src, obj, extra), check=True)


def build(verbose: bool = False, save_temps_dir: str | None = None) -> str:
    """Compile every HIP/C++ source and link libmgs.so (always rebuilds)."""
    with tempfile.TemporaryDirectory(prefix="mgs_build_") as tmp:
        jobs = []
        for name, oname, flags in SOURCES:
            src = os.path.join(CSRC, name)
            obj = os.path.join(tmp, oname + ".o")
            extra = list(flags)
            if save_temps_dir:
                os.makedirs(save_temps_dir, exist_ok=True)
                extra += ["-save-temps=obj", "-o", obj]
            jobs.append((src, obj, extra, oname))

        def run(job):
            src, obj, extra, oname = job
            if verbose:
                print("[build]", oname, flush=True)
            _compile(src, obj, extra)
            return obj

        with concurrent.futures.ThreadPoolExecutor(max_workers=max(1, JOBS)) as pool:
            objs = list(pool.map(run, jobs))
        out_tmp = LIB + ".tmp%d" % os.getpid()
        subprocess.run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", out_tmp, *objs],
                       check=True)
        os.replace(out_tmp, LIB)
        if not save_temps_dir:
            os.makedirs(OBJ_DIR, exist_ok=True)
            for obj in objs:
                shutil.copyfile(obj, os.path.join(OBJ_DIR, os.path.basename(obj)))
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
