"""Pin strength: plausible mistakes planted in a copy of the oracle (on the
CPU) must each make the pin suite fail.  Nothing here touches a GPU or the
HIP path; the mutant libraries live in a temporary directory."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "moe_oracle.c")

# (name, text in moe_oracle.c, replacement)
MUTANTS = [
    ("sigmoid sign", "s[e] = 1.0 / (1.0 + exp(-l));", "s[e] = 1.0 / (1.0 + exp(l));"),
    ("router row/column swapped", "l += x_at(sh, x, t, j) * (double)wr[(int64_t)e * d + j];",
     "l += x_at(sh, x, t, j) * (double)wr[(int64_t)j * E + e % d];"),
    ("bias ignored in choice", "v32[e] = (float)s[e] + bias[e];", "v32[e] = (float)s[e];"),
    ("weights from biased score", "for (int j = 0; j < k; ++j) wgt[j] = s[idx[j]] / sum;",
     "for (int j = 0; j < k; ++j) wgt[j] = (s[idx[j]] + bias[idx[j]]) / sum;"),
    ("ties to higher id", "if (!taken[e] && (best < 0 || v32[e] > v32[best])) best = e;",
     "if (!taken[e] && (best < 0 || v32[e] >= v32[best])) best = e;"),
    ("silu sign", "hbuf[n] = ug / (1.0 + exp(-ug)) * uu;", "hbuf[n] = ug / (1.0 + exp(ug)) * uu;"),
    ("gate/up swapped", "hbuf[n] = ug / (1.0 + exp(-ug)) * uu;", "hbuf[n] = uu / (1.0 + exp(-uu)) * ug;"),
    ("weight transposed", "int64_t i = (g * N + n) * K + j;", "int64_t i = (g * K + j) * N + n;"),
    ("shared expert dropped", "        ffn_row(sh, shared, 0, a, acc, h);\n",
     "        ffn_row(sh, shared, 0, a, acc, h);\n        for (int64_t n = 0; n < d; ++n) acc[n] = 0.0;\n"),
    ("bias step sign flipped", "float sg = diff > 0 ? 1.0f : (diff < 0 ? -1.0f : 0.0f);",
     "float sg = diff > 0 ? -1.0f : (diff < 0 ? 1.0f : 0.0f);"),
    ("sign(0) moves the bias", "float sg = diff > 0 ? 1.0f : (diff < 0 ? -1.0f : 0.0f);",
     "float sg = diff >= 0 ? 1.0f : -1.0f;"),
    ("unstable dispatch", "    for (int64_t f = 0; f < A; ++f) {\n        int e = idx[f];",
     "    for (int64_t f = A - 1; f >= 0; --f) {\n        int e = idx[f];"),
    ("h not rounded to bf16", "for (int i = 0; i < n; ++i) h[i] = bf16_round(h[i]);", "(void)0;"),
    ("y_perm not rounded", "return sh->wt == OR_F32 ? (double)(float)v : bf16_round(v);", "return v;"),
    ("tile scale off", "float t = amax / 448.0f;", "float t = amax / 240.0f;"),
    ("E8M0 bias off by one", "ldexp(1.0, (int)e - 127)", "ldexp(1.0, (int)e - 126)"),
    ("E8M0 encoder off by one", "return (uint8_t)(ex - 1 + 127);", "return (uint8_t)(ex + 127);"),
    ("tile scale not a power of two", "if (b & 0x7FFFFFu) b = (b & 0xFF800000u) + 0x800000u; /* next power of two */",
     "(void)0;"),
    ("gap off by one", "if (r == k) k1th = v[best];", "if (r == k - 1) k1th = v[best];"),
    ("bf16 rounding truncates", "if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u))) upper += 1u;", "(void)lower;"),
    ("e4m3 ties away from zero", "else c = (lo & 1) ? hi : lo;", "else c = hi;"),
]


# mistakes in the backward, against the backward pins
BACKWARD_MUTANTS = [
    ("silu derivative term dropped", "dug[i] = dh * uu * sg * (1.0 + ug * (1.0 - sg));", "dug[i] = dh * uu * sg;"),
    ("gate/up gradients swapped", "dug[i] = dh * uu * sg * (1.0 + ug * (1.0 - sg));\n        duu[i] = dh * ug * sg;",
     "duu[i] = dh * uu * sg * (1.0 + ug * (1.0 - sg));\n        dug[i] = dh * ug * sg;"),
    ("router gradient not renormalised", "const double ds = (dgv[j] - gdg) / ssum;", "const double ds = dgv[j] / ssum;"),
    ("sigmoid derivative dropped", "dl[t * k + j] = ds * s[j] * (1.0 - s[j]);", "dl[t * k + j] = ds;"),
    ("routed gradient not scaled by g", "dyr[n] = gj * (double)dy[t * d + n];", "dyr[n] = (double)dy[t * d + n];"),
    ("down gradient transposed", "dw[n * I + i] += ry[f * d + n] * rh[f * I + i];",
     "dw[n * I + i] += ry[f * d + (n * I + i) % d] * rh[f * I + (n * I + i) / d % I];"),
    ("router input gradient dropped", "acc[n] += dl[t * k + j] * (double)wr[(int64_t)e * d + n];", "(void)e;"),
    ("shared input gradient dropped",
     "fp8 ? sraw + t * 3 * I : NULL);\n        for (int64_t n = 0; n < d; ++n) acc[n] += da[n];",
     "fp8 ? sraw + t * 3 * I : NULL);"),
]


# mistakes in the e4m3 backward's quantisation points, against its pins
FP8_BACKWARD_MUTANTS = [
    ("weight gradient reads unquantised x", "quant_cols(gx, nr, d);", "(void)gx;"),
    ("weight gradient reads unquantised h", "quant_cols(gh, nr, I);", "(void)gh;"),
    ("weight-gradient groups of 64 rows",
     "for (int64_t g0 = 0; g0 < n; g0 += 128) {\n        const int nr = (int)(n - g0 < 128 ? n - g0 : 128);",
     "for (int64_t g0 = 0; g0 < n; g0 += 64) {\n        const int nr = (int)(n - g0 < 64 ? n - g0 : 64);"),
    ("output gradient not quantised for the data gradient", "round_to_gemm_input(sh->wt, dyr, (int)d);",
     "(void)0;"),
    ("weight gradient reads the row-quantised output gradient",
     "if (fp8)\n                for (int64_t n = 0; n < d; ++n) ryr[f * d + n] = dyr[n];\n            round_to_gemm_input(sh->wt, dyr, (int)d);",
     "round_to_gemm_input(sh->wt, dyr, (int)d);\n            if (fp8)\n                for (int64_t n = 0; n < d; ++n) ryr[f * d + n] = dyr[n];"),
]


def _run_pins(tmp_path, old, new, pins):
    src = open(SRC).read()
    assert src.count(old) >= 1, "mutation site not found"
    mut = src.replace(old, new, 1)
    c = tmp_path / "mut.c"
    c.write_text(mut)
    so = tmp_path / "libmut.so"
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fno-fast-math", "-ffp-contract=off", "-shared",
                           "-fPIC", "-o", str(so), str(c), "-lm"])
    env = dict(os.environ, MOE_ORACLE_LIB=str(so), OMP_NUM_THREADS="2")
    return subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                           os.path.join(ROOT, "tests", pins)],
                          cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)


@pytest.mark.parametrize("name,old,new", BACKWARD_MUTANTS, ids=[m[0] for m in BACKWARD_MUTANTS])
def test_backward_pins_catch_mutant(tmp_path, name, old, new):
    r = _run_pins(tmp_path, old, new, "test_oracle_backward_pins.py")
    assert r.returncode != 0, f"mutant '{name}' survived the backward pins:\n{r.stdout[-2000:]}"


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pin_suite_catches_mutant(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation site for '{name}' not found"
    mut = src.replace(old, new, 1)
    c = tmp_path / "mut.c"
    c.write_text(mut)
    so = tmp_path / "libmut.so"
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fno-fast-math", "-ffp-contract=off", "-shared",
                           "-fPIC", "-o", str(so), str(c), "-lm"])
    env = dict(os.environ, MOE_ORACLE_LIB=str(so), OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"mutant '{name}' survived the pins:\n{r.stdout[-2000:]}"


@pytest.mark.parametrize("name,old,new", FP8_BACKWARD_MUTANTS, ids=[m[0] for m in FP8_BACKWARD_MUTANTS])
def test_fp8_backward_pins_catch_mutant(tmp_path, name, old, new):
    r = _run_pins(tmp_path, old, new, "test_oracle_backward_fp8_pins.py")
    assert r.returncode != 0, f"mutant '{name}' survived the e4m3 backward pins:\n{r.stdout[-2000:]}"
