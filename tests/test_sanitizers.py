"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

- The oracle (oracle/oracle.c) built with both and loaded by the whole CPU test
  suite (ORACLE_SANITIZE=1, gcc's ASan runtime preloaded into the interpreter).
- The host code of the HIP library (argument validation, dispatch, workspace
  and scratch bookkeeping) built with both and loaded by the ABI tests, which
  drive every validation path (TA_LIBRARY names that build; clang's ASan runtime
  preloaded). The GPU code of that build is compiled as usual and not run here.
- Two mistakes planted in a copy of oracle.c, an out-of-bounds write and an
  over-wide shift, show that such runs do abort on what they are meant to catch.
Every finding aborts the run (-fno-sanitize-recover=all), so a clean exit means
no report.
"""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GCC_ASAN = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
HAVE_GCC_ASAN = os.path.isabs(GCC_ASAN) and os.path.exists(GCC_ASAN)
REPORT_MARKS = ("ERROR: AddressSanitizer", "runtime error:", "SUMMARY: UndefinedBehaviorSanitizer")


def _run(cmd, env_extra, timeout=900):
    env = dict(os.environ)
    env.update(env_extra)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0"
    return subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=timeout)


@pytest.mark.skipif(not HAVE_GCC_ASAN, reason="gcc's AddressSanitizer runtime is not installed")
def test_cpu_suite_with_sanitized_oracle():
    r = _run([sys.executable, "-m", "pytest", "tests", "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider",
              "--ignore", os.path.join("tests", "test_sanitizers.py")],
             {"ORACLE_SANITIZE": "1", "LD_PRELOAD": GCC_ASAN})
    text = r.stdout + r.stderr
    assert r.returncode == 0, text[-4000:]
    assert not any(m in text for m in REPORT_MARKS), text[-4000:]
    assert os.path.exists(os.path.join(ROOT, "oracle", "liboracle_asan.so"))


def test_abi_validation_with_sanitized_host_code():
    from softmax_tree_reduction_amd import _build
    try:
        _build.hipcc()
        runtime = _build.asan_runtime()
    except RuntimeError as e:
        pytest.skip(str(e))
    lib = _build.build_sanitized()
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True, check=True).stdout
    assert "__ubsan_handle" in syms and "__asan_report" in syms, "the host code is not instrumented"
    r = _run([sys.executable, "-m", "pytest", os.path.join("tests", "test_abi.py"), "-q", "-x",
              "-p", "no:cacheprovider"],
             {"TA_LIBRARY": lib, "LD_PRELOAD": runtime})
    text = r.stdout + r.stderr
    assert r.returncode == 0, text[-4000:]
    assert " passed" in text and " failed" not in text
    assert not any(m in text for m in REPORT_MARKS), text[-4000:]


PLANTED = [
    # qd holds d doubles; writing one more overruns the heap block
    ("out of bounds", "for (int64_t c = 0; c < d; ++c) qd[c] = load_elem(q, dtype, qoff + c);",
     "for (int64_t c = 0; c <= d; ++c) qd[c] = load_elem(q, dtype, qoff + c);", "AddressSanitizer"),
    # a shift by d = 64 bits of a 32-bit int
    ("shift", "const int64_t qoff = (b * Hq + h) * d;",
     "const int64_t qoff = (b * Hq + h) * d + (int64_t)((1 << (int)d) & 0);", "runtime error"),
]

_CALL = """
import ctypes, sys
import numpy as np
lib = ctypes.CDLL(sys.argv[1])
B, Hq, Hkv, N, d = 1, 2, 1, 5, 64
q = np.ones((B, Hq, d), np.float32); k = np.ones((B, Hkv, N, d), np.float32); v = np.ones_like(k)
out = np.zeros((B * Hq, d)); lse = np.zeros(B * Hq)
p = lambda a: a.ctypes.data_as(ctypes.c_void_p)
lib.oracle_decode.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int] + [ctypes.c_int64] * 5 + \\
    [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
print("rc", lib.oracle_decode(p(q), p(k), p(v), 0, B, Hq, Hkv, N, d, None, 0, -1, None, B * Hq, p(out), p(lse)))
"""


@pytest.mark.skipif(not HAVE_GCC_ASAN, reason="gcc's AddressSanitizer runtime is not installed")
@pytest.mark.parametrize("name,old,new,mark", PLANTED, ids=[p[0] for p in PLANTED])
def test_planted_mistakes_abort_the_sanitized_oracle(tmp_path, name, old, new, mark):
    src = open(os.path.join(ROOT, "oracle", "oracle.c")).read()
    assert old in src
    path = tmp_path / "planted.c"
    path.write_text(src.replace(old, new))
    lib = tmp_path / "libplanted.so"
    subprocess.run(["gcc", "-O1", "-fPIC", "-shared", "-std=c11", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", str(path), "-o", str(lib), "-lm"],
                   check=True)
    r = _run([sys.executable, "-c", _CALL, str(lib)], {"LD_PRELOAD": GCC_ASAN}, timeout=120)
    assert r.returncode != 0 and mark in r.stderr, f"planted {name} was not reported: {r.stderr[-2000:]}"
