"""The oracle pins must catch plausible slips in the oracle.

Each case compiles a copy of oracle/oracle.c with one planted mistake (on the
CPU, into a temporary directory), swaps it in for the real oracle library and
runs the pin tests of test_oracle_pins.py against it.  At least one pin must
fail for every mutant; a mutant that survives means the pins have a hole.
"""
import ctypes
import os
import subprocess
import tempfile

import pytest

import oracle
from tests import test_oracle_pins as pins
from tests import test_oracle_pins_linear as lpins
from tests import test_oracle_pins_mingru as mpins
from tests import test_oracle_pins_givens as gpins
from tests import test_oracle_pins_delta as dpins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

# (name, original text, mutated text); each original must occur exactly once
MUTANTS = [
    ("log_fwd drops b", "hp = exp(la[i]) * hp + exp(lb[i]);", "hp = exp(la[i]) * hp;"),
    ("log_fwd sign", "hp = exp(la[i]) * hp + exp(lb[i]);", "hp = exp(la[i]) * hp - exp(lb[i]);"),
    ("log_bwd uses a_t not a_{t+1}", "g = dh[i] + a_next * g;\n                double a = exp(la[i]);",
     "double a = exp(la[i]);\n                g = dh[i] + a * g;"),
    ("log_bwd h_t for h_{t-1}", "dla[i] = g * a * hs[t];", "dla[i] = g * a * hs[t + 1];"),
    ("log_bwd drops b in dlb", "dlb[i] = g * exp(lb[i]);", "dlb[i] = g;"),
    ("log_bwd dlh0 sign", "dlh0[b * d + c] = (T > 0) ? g * a_next * hs[0] : 0.0;",
     "dlh0[b * d + c] = (T > 0) ? -g * a_next * hs[0] : 0.0;"),
    ("linear_fwd drops b", "hp = a[i] * hp + bv[i];", "hp = a[i] * hp;"),
    ("linear_bwd uses a_t not a_{t+1}", "g = dh[i] + a_next * g;\n                da[i] = g * hs[t];",
     "g = dh[i] + a[i] * g;\n                da[i] = g * hs[t];"),
    ("linear_bwd h_t for h_{t-1}", "da[i] = g * hs[t];", "da[i] = g * hs[t + 1];"),
    ("linear_bwd dh0 drops a_1", "dh0[b * d + c] = (T > 0) ? a_next * g : 0.0;",
     "dh0[b * d + c] = (T > 0) ? g : 0.0;"),
    ("mingru_fwd b uses a not 1 - a", "hp = a * hp + (1.0 - a) * gpos(x[i]);", "hp = a * hp + a * gpos(x[i]);"),
    ("mingru_bwd dk drops h_{t-1}", "dk[i] = g * a * (1.0 - a) * (gpos(x[i]) - hs[t]);",
     "dk[i] = g * a * (1.0 - a) * gpos(x[i]);"),
    ("mingru_bwd dx uses a not 1 - a", "dx[i] = g * (1.0 - a) * gpos_d(x[i]);", "dx[i] = g * a * gpos_d(x[i]);"),
    ("mingru_bwd dx0 drops g'", "dx0[b * d + c] = (T > 0) ? g * a_next * gpos_d(x0[b * d + c]) : 0.0;",
     "dx0[b * d + c] = (T > 0) ? g * a_next : 0.0;"),
    ("givens mesh rotation sign", "M[i * k + col] = c * xi - s * xj;\n                    M[j * k + col] = s * xi + c * xj;",
     "M[i * k + col] = c * xi + s * xj;\n                    M[j * k + col] = -s * xi + c * xj;"),
    ("givens mesh derivative sign", "M[i * k + col] = -s * xi - c * xj;", "M[i * k + col] = -s * xi + c * xj;"),
    ("givens ds drops sigmoid'", "dsg[blkid] = sig * (1.0 - sig) * acc;", "dsg[blkid] = sig * acc;"),
    ("givens dtheta drops the gate", "dtheta[blkid * na + rho] = sig * a2;", "dtheta[blkid * na + rho] = a2;"),
    ("affine_fwd transposed A", "for (int64_t c = 0; c < k; ++c) s += At[r * k + c] * cur[c];",
     "for (int64_t c = 0; c < k; ++c) s += At[c * k + r] * cur[c];"),
    ("affine_bwd A not A^T", "for (int64_t r = 0; r < k; ++r) s += At[r * k + c] * g[r];",
     "for (int64_t r = 0; r < k; ++r) s += At[c * k + r] * g[r];"),
    ("affine_bwd h_t for h_{t-1}", "dAt[r * k + c] = g[r] * hs[t * k + c];",
     "dAt[r * k + c] = g[r] * hs[(t + 1) * k + c];"),
    ("affine_bwd dA transposed", "dAt[r * k + c] = g[r] * hs[t * k + c];",
     "dAt[c * k + r] = g[r] * hs[t * k + c];"),
    ("cumprod_fwd P A order", "for (int64_t m = 0; m < k; ++m) s += At[r * k + m] * cur[m * k + c];",
     "for (int64_t m = 0; m < k; ++m) s += cur[r * k + m] * At[m * k + c];"),
    ("cumprod_bwd G P not G P^T", "s += G[r * k + m] * Ps[t * kk + c * k + m];",
     "s += G[r * k + m] * Ps[t * kk + m * k + c];"),
    ("cumprod_bwd A not A^T", "s += At[m * k + r] * G[m * k + c];", "s += At[r * k + m] * G[m * k + c];"),
    ("delta drops beta", "double e = bt * (vt[r] - p[r]);", "double e = (vt[r] - p[r]);"),
    ("delta correction sign", "double e = bt * (vt[r] - p[r]);", "double e = bt * (vt[r] + p[r]);"),
    ("delta reads with q", "for (int64_t c = 0; c < dk; ++c) acc += S[r * dk + c] * kt[c];",
     "for (int64_t c = 0; c < dk; ++c) acc += S[r * dk + c] * qt[c];"),
    ("delta writes along q", "for (int64_t c = 0; c < dk; ++c) S[r * dk + c] += e * kt[c];",
     "for (int64_t c = 0; c < dk; ++c) S[r * dk + c] += e * qt[c];"),
    ("delta output from S_{t-1}",
     "            for (int64_t r = 0; r < dv; ++r) {\n                double e = bt * (vt[r] - p[r]);\n"
     "                for (int64_t c = 0; c < dk; ++c) S[r * dk + c] += e * kt[c];\n            }\n"
     "            for (int64_t r = 0; r < dv; ++r) {\n                double acc = 0.0;\n"
     "                for (int64_t c = 0; c < dk; ++c) acc += S[r * dk + c] * qt[c];\n"
     "                o[(b * T + t) * dv + r] = acc;\n            }\n",
     "            for (int64_t r = 0; r < dv; ++r) {\n                double acc = 0.0;\n"
     "                for (int64_t c = 0; c < dk; ++c) acc += S[r * dk + c] * qt[c];\n"
     "                o[(b * T + t) * dv + r] = acc;\n            }\n"
     "            for (int64_t r = 0; r < dv; ++r) {\n                double e = bt * (vt[r] - p[r]);\n"
     "                for (int64_t c = 0; c < dk; ++c) S[r * dk + c] += e * kt[c];\n            }\n"),
]

PINS = [
    pins.test_golden_log_scan,
    pins.test_golden_block_affine,
    pins.test_golden_block_cumprod,
    lambda: pins.test_log_constant_coefficients_geometric(0.7, 0.3, 2.0),
    pins.test_block_constant_coefficients_geometric,
    pins.test_log_gradients_finite_difference,
    pins.test_block_affine_gradients_finite_difference,
    pins.test_block_cumprod_gradients_finite_difference,
    pins.test_block_affine_brute_force_products,
    pins.test_block_cumprod_brute_force_products,
    lpins.test_golden_linear_scan,
    lambda: lpins.test_constant_coefficients_geometric(-0.8, 1.5, -1.0),
    lpins.test_gradients_finite_difference,
    mpins.test_golden_mingru_cell,
    mpins.test_gradients_finite_difference,
    gpins.test_golden_k2,
    gpins.test_matrices_match_numpy_mesh,
    gpins.test_gradients_finite_difference,
    dpins.test_golden_delta_rule,
    dpins.test_closed_form_householder_products,
    dpins.test_unit_key_full_write,
]


def _build(src_text, out_dir):
    c = os.path.join(out_dir, "mut.c")
    so = os.path.join(out_dir, "libmut.so")
    with open(c, "w") as f:
        f.write(src_text)
    subprocess.run(["gcc", "-O1", "-std=c99", "-shared", "-fPIC", "-o", so, c, "-lm"], check=True)
    return so


@pytest.mark.parametrize("name,orig,mut", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, orig, mut, monkeypatch):
    text = open(SRC).read()
    assert text.count(orig) == 1, f"mutation site not unique for {name!r}"
    oracle._load()  # make sure the real library and its signatures are set up
    real = oracle._lib
    with tempfile.TemporaryDirectory() as tmp:
        lib = ctypes.CDLL(_build(text.replace(orig, mut), tmp))
        for fname in ("oracle_log_fwd", "oracle_log_bwd", "oracle_linear_fwd", "oracle_linear_bwd",
                      "oracle_mingru_fwd", "oracle_mingru_bwd", "oracle_givens_fwd", "oracle_givens_bwd",
                      "oracle_block_affine_fwd",
                      "oracle_block_affine_bwd", "oracle_block_matrix_fwd", "oracle_block_matrix_bwd",
                      "oracle_delta_fwd"):
            fn, ref = getattr(lib, fname), getattr(real, fname)
            fn.argtypes, fn.restype = ref.argtypes, ref.restype
        monkeypatch.setattr(oracle, "_lib", lib)
        caught = []
        for pin in PINS:
            try:
                pin()
            except AssertionError:
                caught.append(getattr(pin, "__name__", "pin"))
        assert caught, f"no pin caught mutant {name!r}"
