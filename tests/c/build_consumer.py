"""Compiles tests/c/abi_consumer.c, a C99 program that uses the library through
include/tree_attn.h only, linked against libtreeattn.so and the HIP runtime."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "abi_consumer.c")
BIN = os.path.join(HERE, "abi_consumer")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def command(out: str = BIN, syntax_only: bool = False) -> list[str]:
    cmd = ["gcc", "-std=c99", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"), SRC]
    if syntax_only:
        return cmd + ["-fsyntax-only"]
    pkg = os.path.join(ROOT, "softmax_tree_reduction_amd")
    return cmd + ["-o", out, "-L", pkg, "-ltreeattn", "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-lm",
                  "-Wl,-rpath,$ORIGIN/../../softmax_tree_reduction_amd", "-Wl,-rpath," + os.path.join(ROCM, "lib")]


def build(out: str = BIN) -> str:
    subprocess.run(command(out), check=True)
    return out


if __name__ == "__main__":
    print(build())
