"""Host sanitizer leg: the C-ABI boundary and the oracle under AddressSanitizer
and UndefinedBehaviorSanitizer.

The boundary's host code (argument validation, overflow-checked sizes,
workspace sizing, geometry) is recompiled with address and undefined-behaviour
checks on the host side only and linked with the GPU objects of the last
build; oracle.c is compiled with the same checks.  The ABI contract tests and
the oracle's pins then run against both in a child process that preloads the
sanitizer runtime, with every report fatal.  A signed overflow in a size
product, an out-of-bounds read in the oracle or a use of freed memory fails
the test.  No GPU is touched: the ABI tests only make calls that fail
validation before any HIP call.
"""
import glob
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from scan_linear_rnns_amd import build as mgs_build  # noqa: E402

CLANG = "/opt/rocm/llvm/bin/clang"
CHECKS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-shared-libsan"]
HOST_CHECKS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
               "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _objects():
    """Objects of the last build other than the boundary's; rebuilt if missing or stale."""
    names = [o for (_, o, _) in mgs_build.SOURCES if o != "mgs_api"]
    paths = [os.path.join(mgs_build.OBJ_DIR, o + ".o") for o in names]
    srcs = glob.glob(os.path.join(mgs_build.CSRC, "*")) + glob.glob(os.path.join(mgs_build.INCLUDE, "*"))
    newest = max(os.path.getmtime(s) for s in srcs)
    if not all(os.path.exists(p) and os.path.getmtime(p) >= newest for p in paths):
        mgs_build.build()
    return paths


@pytest.mark.skipif(not os.path.exists(CLANG), reason="ROCm clang not installed")
def test_abi_and_oracle_under_sanitizers():
    rt = subprocess.run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                        text=True, check=True).stdout.strip()
    assert os.path.exists(rt), rt
    objs = _objects()
    with tempfile.TemporaryDirectory(prefix="mgs_san_") as tmp:
        api = os.path.join(tmp, "mgs_api_san.o")
        cmd = mgs_build.compile_cmd(os.path.join(mgs_build.CSRC, "mgs_api.cpp"), api, ["-g", *HOST_CHECKS])
        subprocess.run(cmd, check=True, capture_output=True)
        lib = os.path.join(tmp, "libmgs_san.so")
        link = [CLANG + "++", "-shared", "-fPIC", *CHECKS, "-o", lib, api, *objs,
                "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"]
        subprocess.run(link, check=True, capture_output=True)
        olib = os.path.join(tmp, "liboracle_san.so")
        subprocess.run([CLANG, "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off", "-std=c99", *CHECKS,
                        "-shared", "-fPIC", "-o", olib, os.path.join(ROOT, "oracle", "oracle.c"), "-lm"],
                       check=True, capture_output=True)
        env = dict(os.environ, LD_PRELOAD=rt, MGS_LIBRARY=lib, MGS_ORACLE_LIBRARY=olib,
                   ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
                   UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
        tests = [os.path.join(ROOT, "tests", t) for t in
                 ("test_abi_cpu.py", "test_oracle_pins.py", "test_oracle_pins_linear.py",
                  "test_oracle_pins_mingru.py", "test_oracle_pins_givens.py", "test_oracle_pins_delta.py")]
        r = subprocess.run([sys.executable, "-m", "pytest", *tests, "-m", "not gpu", "-q", "-x",
                            "-p", "no:cacheprovider"], env=env, cwd=ROOT, capture_output=True, text=True,
                           timeout=600)
        out = r.stdout + r.stderr
        assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
        assert r.returncode == 0, out[-4000:]
        assert " passed" in out, out[-2000:]
