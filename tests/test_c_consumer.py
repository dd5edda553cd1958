"""The C ABI from plain C: include/tree_attn.h compiles as strict C99 and as C++,
and (on a GPU) a C99 program that uses nothing but the header, the library and
the HIP runtime's C API checks closed-form results (tests/c/abi_consumer.c)."""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
sys.path.insert(0, os.path.join(HERE, "c"))
import build_consumer  # noqa: E402


@pytest.mark.parametrize("lang", [["gcc", "-x", "c", "-std=c99"], ["g++", "-x", "c++", "-std=c++17"]])
def test_header_compiles_alone(lang, tmp_path):
    src = tmp_path / "inc.c"
    src.write_text('#include "tree_attn.h"\nint main(void) { ta_tensor t; (void)t; return TA_OK; }\n')
    subprocess.run([*lang, "-Wall", "-Wextra", "-pedantic", "-Werror", "-I", os.path.join(ROOT, "include"),
                    "-fsyntax-only", str(src)], check=True)


def test_consumer_compiles():
    subprocess.run(build_consumer.command(syntax_only=True), check=True)


@pytest.mark.gpu
def test_consumer_runs_on_the_gpu():
    if not os.path.exists(build_consumer.BIN):
        build_consumer.build()
    r = subprocess.run([build_consumer.BIN], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0, r.stderr
    assert "all checks passed" in r.stdout
