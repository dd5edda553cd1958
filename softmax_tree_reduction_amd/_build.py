"""Compile the HIP sources of this package into libtreeattn.so (gfx950)."""
from __future__ import annotations

import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
LIB = os.path.join(HERE, "libtreeattn.so")
SOURCES = ["api.hip", "partial.hip", "combine.hip", "probe.hip"]
ARCH = "gfx950"

# Packed fp32 instructions stay off: all float math is issued as scalar VALU ops.
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


# A copy of the library whose host code (argument validation, dispatch, workspace)
# is instrumented with AddressSanitizer and UndefinedBehaviorSanitizer; the GPU code
# is built as usual. A process using it needs clang's ASan runtime preloaded.
SAN_LIB = os.path.join(HERE, "_build_san", "libtreeattn_san.so")
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-sanitize-recover=all",
             "-Xarch_host", "-fno-omit-frame-pointer", "-shared-libsan"]


def asan_runtime() -> str:
    """Path of the ASan runtime of hipcc's clang (to preload into a process that
    loads the sanitized library)."""
    res = subprocess.run([hipcc(), "--print-file-name=libclang_rt.asan-x86_64.so"], check=True,
                         capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(res) or not os.path.exists(res):
        raise RuntimeError(f"clang ASan runtime not found ({res!r})")
    return res


def build_sanitized(verbose: bool = False) -> str:
    """Build SAN_LIB: host code under ASan and UBSan (any finding aborts)."""
    return build(verbose, extra_flags=SAN_FLAGS, out=SAN_LIB, objdir=os.path.join(HERE, "_build_san"),
                 link_flags=SAN_FLAGS)


def build(verbose: bool = False, extra_flags: list[str] | None = None, out: str = LIB,
          objdir: str | None = None, link_flags: list[str] | None = None) -> str:
    """Compile every source, link the shared library (in place by default), return its path."""
    cc = hipcc()
    objdir = objdir or os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    flags = HIP_FLAGS + list(extra_flags or [])

    def compile_one(src: str) -> str:
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        cmd = [cc, *flags, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        return obj

    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = out + f".tmp{os.getpid()}"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *(link_flags or []), *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
