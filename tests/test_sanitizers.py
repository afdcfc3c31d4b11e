"""Memory and undefined-behaviour checks of the host code: the CPU oracle
and the C ABI library's host side.

The oracle (oracle/moe_oracle.c) is built a second time with
AddressSanitizer and UndefinedBehaviorSanitizer (gcc, any error aborts) and
every exported entry point runs on small seeded inputs in a child process
that preloads the ASan runtime: the forward (route, dispatch, bias step,
routed FFN, combine, whole forward) in f32, bf16 and e4m3, the e4m3 row
quantiser, and the backward (all gradients, the single-expert and the
dx-only forms, the shared expert's column-restricted form).  Out-of-bounds
accesses, use-after-free and undefined arithmetic (signed overflow, bad
shifts, misaligned loads) fail the test with the sanitizer's report.

The C ABI's host code (argument and shape validation, workspace sizing,
status strings: csrc/moe_api.hip) is likewise rebuilt with ASan and UBSan on
its host pass only (the device code is the normal build's) and the library
tests of tests/test_abi.py, which run on the CPU and never reach a kernel,
run against that build.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import sys
sys.path.insert(0, ROOT)
import numpy as np
import oracle
import synth

oracle.set_threads(2)
for name, act, wt, T, d, I in (("f32", "f32", "f32", 9, 128, 64), ("bf16", "bf16", "bf16", 11, 128, 128),
                               ("e4m3", "bf16", "e4m3", 10, 256, 128)):
    cfg = synth.CONFIGS[2].with_(name="san-" + name, seed=5, T=T, d=d, I=I, act=act, wt=wt)
    inp = synth.make_inputs(cfg)
    sh = oracle.shape_of(cfg)
    idx, g, gap, s = oracle.route(sh, inp["x"], inp["wr"], inp["bias"], want_s=True)
    idx2, g2, gap2 = oracle.choose(s, inp["bias"], cfg.k)[:3]
    assert np.array_equal(idx, idx2)
    counts, offsets, row_src, row_of = oracle.dispatch(idx, cfg.E)
    oracle.bias_update(inp["bias"], counts, cfg.k, cfg.T, cfg.gamma)
    a = np.ascontiguousarray(inp["x"][row_src // cfg.k])
    a_sc = None
    if wt == "e4m3":
        q, a_sc = oracle.quant_e4m3_rows(inp["x"])
        a, a_sc = np.ascontiguousarray(q[row_src // cfg.k]), np.ascontiguousarray(a_sc[row_src // cfg.k])
    yp = oracle.expert_ffn(sh, inp["experts"], offsets, a, a_sc)
    yp_rows = oracle.expert_ffn(sh, inp["experts"], offsets, a, a_sc, rows=np.array([0, T * 8 - 1], np.int32))
    oracle.combine(sh, inp["shared"], inp["x"], yp, row_of, g)
    oracle.forward(sh, inp["x"], inp["wr"], inp["bias"], inp["experts"], inp["shared"])
    oracle.forward(sh, inp["x"], inp["wr"], inp["bias"], inp["experts"], inp["shared"], np.array([T - 1], np.int32))
    dy = synth.normal(cfg.seed, synth.TID_AUX, (T, d), 1.0, "f32")
    if act == "bf16":
        oracle.backward(sh, inp["x"], inp["wr"], idx, inp["experts"], inp["shared"], dy)
        oracle.backward(sh, inp["x"], inp["wr"], idx, inp["experts"], inp["shared"], dy, weight_grads=False)
        oracle.backward(sh, inp["x"], inp["wr"], idx, inp["experts"], inp["shared"], dy,
                        weight_grads=int(idx[0, 0]))
        oracle.backward_shared_cols(sh, inp["x"], inp["shared"], dy, np.array([0, I - 1]))
    print("ok", name, flush=True)
"""


def _asan_runtime():
    r = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True)
    p = r.stdout.strip()
    return p if r.returncode == 0 and os.path.isabs(p) and os.path.exists(p) else None


def test_oracle_clean_under_asan_and_ubsan(tmp_path):
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    lib = str(tmp_path / "liboracle_san.so")
    # the oracle's own build line, plus the sanitizers (host C code only)
    subprocess.check_call(["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fopenmp", "-fno-fast-math",
                           "-ffp-contract=off", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                           "-shared", "-fPIC", "-o", lib, os.path.join(ROOT, "oracle", "moe_oracle.c"), "-lm"])
    env = dict(os.environ, LD_PRELOAD=rt, MOE_ORACLE_LIB=lib, OMP_NUM_THREADS="2",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([sys.executable, "-c", CHILD.replace("ROOT", repr(ROOT))], env=env, capture_output=True,
                       text=True, timeout=600)
    assert r.returncode == 0, f"sanitizer run failed (exit {r.returncode}):\n{r.stdout[-2000:]}\n{r.stderr[-6000:]}"
    assert [ln for ln in r.stdout.splitlines() if ln.startswith("ok ")] == ["ok f32", "ok bf16", "ok e4m3"]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-6000:]


ABI_CHILD = r"""
import sys
sys.path.insert(0, ROOT)
from sparse_expert_routing_amd import _lib
_lib.load(LIB)
import pytest
sys.exit(pytest.main(["-q", "-p", "no:cacheprovider", "-m", "not gpu", ROOT + "/tests/test_abi.py"]))
"""


def _clang_asan_runtime(hipcc):
    r = subprocess.run([hipcc, "--print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    p = r.stdout.strip()
    if r.returncode == 0 and os.path.isabs(p) and os.path.exists(p):
        return p
    r = subprocess.run([hipcc, "--print-resource-dir"], capture_output=True, text=True)
    p = os.path.join(r.stdout.strip(), "lib", "linux", "libclang_rt.asan-x86_64.so")
    return p if r.returncode == 0 and os.path.exists(p) else None


def test_abi_host_code_clean_under_asan_and_ubsan(tmp_path):
    sys.path.insert(0, ROOT)
    from sparse_expert_routing_amd import build as B
    if not os.path.exists(B.HIPCC):
        pytest.skip("hipcc is not installed")
    rt = _clang_asan_runtime(B.HIPCC)
    if rt is None:
        pytest.skip("the compiler's AddressSanitizer runtime is not installed")
    objs = []
    for src in B.sources():
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        if os.path.basename(src) == "moe_api.hip":
            # host pass only: every sanitizer flag sits behind -Xarch_host
            extra = ["-O1", "-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                     "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
            subprocess.check_call([B.HIPCC, *B.FLAGS, *extra, "-c", src, "-o", obj])
        else:
            prebuilt = os.path.join(B.BUILD, os.path.basename(src) + ".o")
            if not os.path.exists(prebuilt):
                pytest.skip("build the library first (its objects are reused)")
            obj = prebuilt
        objs.append(obj)
    lib = str(tmp_path / "libmoe_san.so")
    subprocess.check_call([B.HIPCC, f"--offload-arch={B.ARCH}", "-shared", "-fPIC", "-Xarch_host",
                           "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-Xarch_host",
                           "-shared-libsan", "-o", lib, *objs])
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1")
    code = ABI_CHILD.replace("ROOT", repr(ROOT)).replace("LIB", repr(lib))
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=600,
                       cwd=str(tmp_path))
    assert r.returncode == 0, f"sanitizer run failed (exit {r.returncode}):\n{r.stdout[-4000:]}\n{r.stderr[-6000:]}"
    assert " passed" in r.stdout and "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
