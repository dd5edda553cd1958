"""CPU oracle for single-query decode attention and the tree merge of partial states.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU
baseline leg may import this package; the product library never does, and
this package imports nothing from it.

Two parts:

* ``decode`` and ``combine`` wrap ``oracle.c``: the plain float64 definition of
  softmax(q K^T / sqrt(d)) V with its log-sum-exp, and the plain definition of
  merging normalised partial states. They use no chunking and no merge operator.
* ``merge``, ``tree_fold`` and the state conversions restate, in numpy float64,
  the merge operator and tree reduction of "Tree Attention Guide: Topology-Aware
  LLM Decoding" (sections "Core Innovation 1: Logarithmic Tree-Based Attention
  Reduction" and "Core Innovation 2: Mathematical Formulation of Online Softmax
  on Trees"), in the page's notation (o, l, m). The tests pin them against the
  plain definitions above.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

F32, BF16 = 0, 1


# ORACLE_SANITIZE=1 builds and loads a copy instrumented with AddressSanitizer and
# UndefinedBehaviorSanitizer (any finding aborts the process). The process must
# then start with gcc's libasan preloaded (LD_PRELOAD), as a non-instrumented
# Python interpreter loads the library.
_SAN_LIB = os.path.join(_HERE, "liboracle_asan.so")
_SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]


def _sanitized() -> bool:
    return os.environ.get("ORACLE_SANITIZE", "") == "1"


def build(force: bool = False) -> str:
    """Compile oracle.c with gcc (float64, OpenMP). Returns the library path."""
    lib = _SAN_LIB if _sanitized() else _LIB
    if force or not os.path.exists(lib) or os.path.getmtime(lib) < os.path.getmtime(_SRC):
        tmp = lib + f".tmp{os.getpid()}"
        subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                        "-Wall", "-Wextra", *(_SAN_FLAGS if _sanitized() else []), _SRC, "-o", tmp, "-lm"],
                       check=True)
        os.replace(tmp, lib)
    return lib


def _load():
    global _lib
    with _lock:
        if _lib is None:
            lib = ctypes.CDLL(build())
            p, i64, i32, dp = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
            lib.oracle_decode.argtypes = [p, p, p, i32, i64, i64, i64, i64, i64, p, i64, i64, p, i64, dp, dp]
            lib.oracle_decode.restype = ctypes.c_int
            lib.oracle_combine.argtypes = [p, p, i64, i64, i64, dp, dp]
            lib.oracle_combine.restype = ctypes.c_int
            lib.oracle_num_threads.restype = ctypes.c_int
            lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
            lib.oracle_set_num_threads.restype = None
            _lib = lib
    return _lib


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """OpenMP threads for later calls (timing only: results do not depend on it)."""
    _load().oracle_set_num_threads(int(n))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:   # bfloat16 bit patterns
        return BF16
    raise TypeError(f"oracle takes float32 or bf16-bits (uint16) arrays, got {a.dtype}")


def decode(q, k, v, seqlens=None, *, t_begin: int = 0, t_end: int = -1, rows=None):
    """Exact decode attention in float64.

    q [B, Hq, d]; k, v [B, Hkv, N, d] (float32, or uint16 bfloat16 bits);
    seqlens int32 [B] or None; the token window [t_begin, t_end) is
    intersected with each sequence; rows = flat ids b*Hq+h to compute (default all).
    Returns (out [n_rows, d] float64, lse [n_rows] float64) -- for the default
    rows, shaped [B, Hq, d] and [B, Hq].
    """
    q, k, v = (np.ascontiguousarray(x) for x in (q, k, v))
    B, Hq, d = q.shape
    Bk, Hkv, N, dk = k.shape
    if k.shape != v.shape or Bk != B or dk != d:
        raise ValueError("shape mismatch between q, k and v")
    code = _dtype_code(q)
    if _dtype_code(k) != code or _dtype_code(v) != code:
        raise TypeError("q, k and v must share a dtype")
    sl = None if seqlens is None else np.ascontiguousarray(seqlens, dtype=np.int32)
    if rows is None:
        sel, n_rows = None, B * Hq
    else:
        sel = np.ascontiguousarray(rows, dtype=np.int64)
        n_rows = sel.size
    out = np.zeros((n_rows, d), dtype=np.float64)
    lse = np.zeros(n_rows, dtype=np.float64)
    rc = _load().oracle_decode(_ptr(q), _ptr(k), _ptr(v), code, B, Hq, Hkv, N, d,
                               None if sl is None else _ptr(sl), int(t_begin), int(t_end),
                               None if sel is None else _ptr(sel), n_rows, _ptr(out), _ptr(lse))
    if rc != 0:
        raise RuntimeError(f"oracle_decode failed with code {rc}")
    if rows is None:
        return out.reshape(B, Hq, d), lse.reshape(B, Hq)
    return out, lse


def combine(partial_o, partial_lse):
    """Merge normalised partial states by definition (log-sum-exp weights), float64.

    partial_o float32 [..., n_parts, d], partial_lse float32 [..., n_parts].
    Returns (out [..., d], lse [...]) in float64.
    """
    po = np.ascontiguousarray(partial_o, dtype=np.float32)
    pl = np.ascontiguousarray(partial_lse, dtype=np.float32)
    lead, (P, d) = po.shape[:-2], po.shape[-2:]
    if pl.shape != lead + (P,):
        raise ValueError("partial_lse shape must be partial_o shape without d")
    rows = int(np.prod(lead, dtype=np.int64)) if lead else 1
    out = np.zeros((rows, d), dtype=np.float64)
    lse = np.zeros(rows, dtype=np.float64)
    rc = _load().oracle_combine(_ptr(po), _ptr(pl), rows, P, d, _ptr(out), _ptr(lse))
    if rc != 0:
        raise RuntimeError(f"oracle_combine failed with code {rc}")
    return out.reshape(lead + (d,)), lse.reshape(lead)


# ----------------------------------------------------------------------------
# The merge operator and the tree reduction, in the page's notation.
#
# A partial state over a token set T is the tuple (o, l, m):
#   m = max_{j in T} s_j,  l = sum_{j in T} exp(s_j - m),  o = sum_{j in T} exp(s_j - m) v_j
# ("Core Innovation 1", step 2). The empty set is (0, 0, -inf).
# ----------------------------------------------------------------------------

def empty_state(d: int):
    return (np.zeros(d, dtype=np.float64), 0.0, -np.inf)


def merge(a, b):
    """The merge operator of "Core Innovation 2" on two (o, l, m) states, float64.

    m_new = max(m_A, m_B); alpha = exp(m_A - m_new); beta = exp(m_B - m_new);
    l_new = alpha l_A + beta l_B; o_new = alpha o_A + beta o_B.
    Reading for empty states (the page does not cover them): when both maxima
    are -inf the formula would take exp(-inf - (-inf)); the union of two empty
    sets is empty, so the result is the empty state.
    """
    o_a, l_a, m_a = a
    o_b, l_b, m_b = b
    m_new = max(m_a, m_b)
    if m_new == -np.inf:
        return empty_state(np.asarray(o_a).shape[-1])
    alpha = np.exp(m_a - m_new)
    beta = np.exp(m_b - m_new)
    l_new = alpha * l_a + beta * l_b
    o_new = alpha * np.asarray(o_a, dtype=np.float64) + beta * np.asarray(o_b, dtype=np.float64)
    return (o_new, l_new, m_new)


def finalize(state):
    """Root normalisation ("Core Innovation 2", final step): O = o / l, and lse = m + ln l."""
    o, l, m = state
    if m == -np.inf or l == 0.0:
        return np.zeros_like(np.asarray(o, dtype=np.float64)), -np.inf
    return np.asarray(o, dtype=np.float64) / l, m + np.log(l)


def from_normalized(o_norm, lse):
    """A normalised state (o/l, m + ln l) as an (o, l, m) tuple: (o/l, 1, lse) is the same state."""
    if lse == -np.inf:
        return empty_state(np.asarray(o_norm).shape[-1])
    return (np.asarray(o_norm, dtype=np.float64), 1.0, float(lse))


def tree_fold(states, arity: int = 2):
    """Reduce states up a tree of the given arity ("Core Innovation 1", step 3).

    At each level, consecutive groups of `arity` nodes are merged left to
    right into their parent; a short last group merges what it has (a lone
    node passes through). Returns (root state, number of levels), where the
    number of levels is ceil(log_arity(P)) for P leaves.
    """
    if arity < 2:
        raise ValueError("arity must be at least 2")
    nodes = list(states)
    if not nodes:
        raise ValueError("no states to reduce")
    levels = 0
    while len(nodes) > 1:
        parents = []
        for i in range(0, len(nodes), arity):
            acc = nodes[i]
            for child in nodes[i + 1:i + arity]:
                acc = merge(acc, child)
            parents.append(acc)
        nodes = parents
        levels += 1
    return nodes[0], levels


def chain_fold(states):
    """Merge states one after another (the sequential order of a ring): P - 1 steps."""
    nodes = list(states)
    acc = nodes[0]
    for s in nodes[1:]:
        acc = merge(acc, s)
    return acc, len(nodes) - 1
