"""Host-side checks of the C ABI: the library loads, exports what
include/tree_attn.h declares, and rejects bad descriptors before touching the
GPU (argument validation runs before any HIP call, so these need no device;
the data pointers below are never dereferenced)."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

import softmax_tree_reduction_amd as ta

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10000  # a 16-byte aligned non-null address; validation never reads it

pytestmark = pytest.mark.skipif(not os.path.exists(ta.library_path()),
                                reason="libtreeattn.so not built")


def declared_functions():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            src = open(os.path.join(ROOT, "include", fn)).read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            names.update(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(ta_\w+)\s*\(", src, flags=re.M))
    return names


def test_exports_every_declared_symbol():
    lib = ta.load_library()
    names = declared_functions()
    assert {"ta_decode", "ta_combine", "ta_combine_k", "ta_combine_chain", "ta_partial", "ta_stream_read",
            "ta_suggest_chunk", "ta_last_error", "ta_version"} <= names
    for n in names:
        assert hasattr(lib, n), f"{n} declared in include/ but not exported"
    assert set(ta.EXPORTS) == names
    assert lib.ta_version() == 1
    assert lib.ta_last_error() is not None


def T(shape, dtype=ta.TA_BF16, stride=None, data=FAKE):
    if stride is None:
        stride, acc = [], 1
        for s in reversed(shape):
            stride.insert(0, acc)
            acc *= s
    return ta.TaTensor.make(data, dtype, shape, stride)


def good(B=2, Hq=8, Hkv=2, N=1000, d=128, dt=ta.TA_BF16):
    return dict(q=T([B, Hq, d], dt), k=T([B, Hkv, N, d], dt), v=T([B, Hkv, N, d], dt),
                out=T([B, Hq, d], ta.TA_F32), lse=T([B, Hq], ta.TA_F32))


def call_decode(a, chunk=256):
    lib = ta.load_library()
    ref = lambda x: None if x is None else ctypes.byref(x)
    rc = lib.ta_decode(ref(a["q"]), ref(a["k"]), ref(a["v"]), None, ref(a["out"]), ref(a.get("lse")), chunk, None)
    return rc, lib.ta_last_error().decode()


def call_partial(a, po, pl, chunk=256):
    lib = ta.load_library()
    rc = lib.ta_partial(ctypes.byref(a["q"]), ctypes.byref(a["k"]), ctypes.byref(a["v"]), None,
                        ctypes.byref(po), ctypes.byref(pl), chunk, None)
    return rc, lib.ta_last_error().decode()


def call_combine(po, pl, n, out, lse):
    lib = ta.load_library()
    ref = lambda x: None if x is None else ctypes.byref(x)
    rc = lib.ta_combine(ref(po), ref(pl), n, ref(out), ref(lse), None)
    return rc, lib.ta_last_error().decode()


@pytest.mark.parametrize("mutate,code,needle", [
    (lambda a: a.update(q=None), ta.TA_ERR_NULL, "q"),
    (lambda a: a.update(out=None), ta.TA_ERR_NULL, "out"),
    (lambda a: setattr(a["k"], "data", None), ta.TA_ERR_NULL, "k"),
    (lambda a: setattr(a["q"], "ndim", 2), ta.TA_ERR_SHAPE, "dimensions"),
    (lambda a: a.update(q=T([2, 6, 128])), ta.TA_ERR_SHAPE, "multiple"),     # 6 % 4 != 0 after k change below
    (lambda a: a.update(v=T([2, 2, 999, 128])), ta.TA_ERR_SHAPE, "differ"),
    (lambda a: a.update(k=T([3, 2, 1000, 128]), v=T([3, 2, 1000, 128])), ta.TA_ERR_SHAPE, "batch"),
    (lambda a: a.update(v=T([2, 2, 1000, 128], ta.TA_F32)), ta.TA_ERR_DTYPE, "dtype"),
    (lambda a: setattr(a["q"], "dtype", 7), ta.TA_ERR_DTYPE, "dtype"),
    (lambda a: a.update(out=T([2, 8, 128], ta.TA_BF16)), ta.TA_ERR_DTYPE, "out"),
    (lambda a: a.update(out=T([2, 8, 64], ta.TA_F32)), ta.TA_ERR_SHAPE, "out"),
    (lambda a: a.update(lse=T([2, 4], ta.TA_F32)), ta.TA_ERR_SHAPE, "lse"),
    (lambda a: a.update(k=T([2, 2, 1000, 128], stride=[256000, 128000, 128, 2])), ta.TA_ERR_STRIDE, "contiguous"),
    (lambda a: a.update(k=T([2, 2, 1000, 128], stride=[257000, 128500, 129, 1])), ta.TA_ERR_STRIDE, "16 bytes"),
    (lambda a: setattr(a["v"], "data", FAKE + 2), ta.TA_ERR_STRIDE, "aligned"),
])
def test_decode_validation(mutate, code, needle):
    a = good()
    if needle == "multiple":
        a = good(Hq=8, Hkv=4)
        a["q"] = T([2, 6, 128])
        a["out"] = T([2, 6, 128], ta.TA_F32)
        a["lse"] = T([2, 6], ta.TA_F32)
        a["k"] = T([2, 4, 1000, 128])
        a["v"] = T([2, 4, 1000, 128])
    else:
        mutate(a)
    rc, msg = call_decode(a)
    assert rc == code, msg
    assert needle in msg


def test_null_data_is_accepted_only_for_tensors_without_elements():
    # an empty cache (N = 0) may come with NULL k and v pointers; validation passes
    # them (on a machine without a GPU the call then fails on the device query)
    a = good(N=0)
    a["k"].data = None
    a["v"].data = None
    rc, msg = call_decode(a)
    assert rc != ta.TA_ERR_NULL, msg
    a = good(N=1)
    a["k"].data = None
    rc, msg = call_decode(a)
    assert rc == ta.TA_ERR_NULL and "k" in msg


def test_decode_unsupported_and_bad_chunk():
    rc, msg = call_decode(good(d=96))
    assert rc == ta.TA_ERR_UNSUPPORTED and "96" in msg
    rc, msg = call_decode(good(), chunk=0)
    assert rc == ta.TA_ERR_ARG and "chunk" in msg
    rc, msg = call_decode(good(B=70000))
    assert rc == ta.TA_ERR_UNSUPPORTED


def test_decode_empty_batch_is_a_no_op():
    # B = 0: valid, nothing to launch
    rc, msg = call_decode(good(B=0))
    assert rc == ta.TA_OK, msg


def test_partial_validation():
    a = good(N=1000)
    # 1000 tokens in chunks of 256 need 4 partial states
    rc, msg = call_partial(a, T([2, 8, 3, 128], ta.TA_F32), T([2, 8, 3], ta.TA_F32))
    assert rc == ta.TA_ERR_SHAPE and "needs 4" in msg
    rc, msg = call_partial(a, T([2, 8, 4, 128], ta.TA_BF16), T([2, 8, 4], ta.TA_F32))
    assert rc == ta.TA_ERR_DTYPE
    rc, msg = call_partial(a, T([2, 8, 4, 128], ta.TA_F32), T([2, 8, 5], ta.TA_F32))
    assert rc == ta.TA_ERR_SHAPE


def test_combine_validation():
    po, pl = T([2, 8, 16, 128], ta.TA_F32), T([2, 8, 16], ta.TA_F32)
    out, lse = T([2, 8, 128], ta.TA_F32), T([2, 8], ta.TA_F32)
    assert call_combine(None, pl, 4, out, lse)[0] == ta.TA_ERR_NULL
    assert call_combine(po, pl, 17, out, lse)[0] == ta.TA_ERR_ARG
    assert call_combine(po, pl, -1, out, lse)[0] == ta.TA_ERR_ARG
    assert call_combine(po, T([2, 8, 15], ta.TA_F32), 4, out, lse)[0] == ta.TA_ERR_SHAPE
    assert call_combine(T([2, 8, 16, 96], ta.TA_F32), pl, 4, T([2, 8, 96], ta.TA_F32), lse)[0] == ta.TA_ERR_UNSUPPORTED
    assert call_combine(po, pl, 4, T([2, 8, 64], ta.TA_F32), lse)[0] == ta.TA_ERR_SHAPE
    assert call_combine(po, pl, 4, out, T([2, 8], ta.TA_BF16))[0] == ta.TA_ERR_DTYPE
    rc, msg = call_combine(T([0, 8, 16, 128], ta.TA_F32), T([0, 8, 16], ta.TA_F32), 4,
                           T([0, 8, 128], ta.TA_F32), T([0, 8], ta.TA_F32))
    assert rc == ta.TA_OK, msg


def call_combine_k(po, pl, n, arity, out, lse):
    lib = ta.load_library()
    ref = lambda x: None if x is None else ctypes.byref(x)
    rc = lib.ta_combine_k(ref(po), ref(pl), n, arity, ref(out), ref(lse), None)
    return rc, lib.ta_last_error().decode()


def test_combine_k_validation():
    po, pl = T([2, 8, 16, 128], ta.TA_F32), T([2, 8, 16], ta.TA_F32)
    out, lse = T([2, 8, 128], ta.TA_F32), T([2, 8], ta.TA_F32)
    for bad in (-1, 0, 1, 17, 1 << 20):
        rc, msg = call_combine_k(po, pl, 4, bad, out, lse)
        assert rc == ta.TA_ERR_ARG and "arity" in msg
    assert call_combine_k(None, pl, 4, 4, out, lse)[0] == ta.TA_ERR_NULL
    assert call_combine_k(po, pl, 17, 4, out, lse)[0] == ta.TA_ERR_ARG
    assert call_combine_k(po, T([2, 8, 15], ta.TA_F32), 4, 4, out, lse)[0] == ta.TA_ERR_SHAPE
    assert call_combine_k(T([2, 8, 16, 96], ta.TA_F32), pl, 4, 8, T([2, 8, 96], ta.TA_F32), lse)[0] == \
        ta.TA_ERR_UNSUPPORTED
    rc, msg = call_combine_k(T([2, 0, 16, 128], ta.TA_F32), T([2, 0, 16], ta.TA_F32), 4, 16,
                             T([2, 0, 128], ta.TA_F32), T([2, 0], ta.TA_F32))
    assert rc == ta.TA_OK, msg


def test_combine_chain_validation():
    lib = ta.load_library()
    ref = lambda x: None if x is None else ctypes.byref(x)
    call = lambda po, pl, n, out, lse: (lib.ta_combine_chain(ref(po), ref(pl), n, ref(out), ref(lse), None),
                                        lib.ta_last_error().decode())
    po, pl = T([2, 8, 16, 128], ta.TA_F32), T([2, 8, 16], ta.TA_F32)
    out, lse = T([2, 8, 128], ta.TA_F32), T([2, 8], ta.TA_F32)
    assert call(None, pl, 4, out, lse)[0] == ta.TA_ERR_NULL
    assert call(po, pl, 17, out, lse)[0] == ta.TA_ERR_ARG
    assert call(po, pl, -1, out, lse)[0] == ta.TA_ERR_ARG
    assert call(po, T([2, 8, 15], ta.TA_F32), 4, out, lse)[0] == ta.TA_ERR_SHAPE
    assert call(T([2, 8, 16, 96], ta.TA_F32), pl, 4, T([2, 8, 96], ta.TA_F32), lse)[0] == ta.TA_ERR_UNSUPPORTED
    assert call(po, pl, 4, out, T([2, 8], ta.TA_BF16))[0] == ta.TA_ERR_DTYPE
    rc, msg = call(T([0, 8, 16, 128], ta.TA_F32), T([0, 8, 16], ta.TA_F32), 4, T([0, 8, 128], ta.TA_F32),
                   T([0, 8], ta.TA_F32))
    assert rc == ta.TA_OK, msg


def test_stream_read_validation():
    lib = ta.load_library()
    vp = ctypes.c_void_p
    call = lambda buf, n, sink: (lib.ta_stream_read(vp(buf), ctypes.c_int64(n), vp(sink), None),
                                 lib.ta_last_error().decode())
    assert call(None, 16, FAKE)[0] == ta.TA_ERR_NULL
    assert call(FAKE, 16, None)[0] == ta.TA_ERR_NULL
    rc, msg = call(FAKE, 24, FAKE)
    assert rc == ta.TA_ERR_ARG and "multiple of 16" in msg
    assert call(FAKE, -16, FAKE)[0] == ta.TA_ERR_ARG
    rc, msg = call(FAKE + 8, 16, FAKE)
    assert rc == ta.TA_ERR_ARG and "aligned" in msg
    assert call(FAKE, 0, FAKE) == (ta.TA_OK, "")


def test_suggest_chunk():
    # the chunks that measured fastest for one 8B-GQA sequence (32 query heads, 8 KV
    # heads: 8 head groups) on 256 compute units give one workgroup per CU each
    for n, want in [(8192, 256), (32768, 1024), (131072, 4096), (1 << 20, 32768)]:
        assert ta.suggest_chunk(1, 32, 8, n, compute_units=256) == want
    assert ta.suggest_chunk(4, 32, 8, 524288, compute_units=256) == 65536
    # the defining property over a grid of shapes: the largest power of two (>= 64,
    # <= n unless n < 64) whose grid still has a workgroup per compute unit
    for B in (1, 3, 32):
        for Hq, Hkv in ((32, 8), (8, 8), (12, 4), (5, 1)):
            g = next(x for x in (8, 4, 2, 1) if (Hq // Hkv) % x == 0)
            rows = B * Hq // g
            for n in (1, 63, 64, 100, 4096, 100000, 1 << 20):
                for cus in (1, 80, 256, 304):
                    c = ta.suggest_chunk(B, Hq, Hkv, n, compute_units=cus)
                    assert c >= 64 and c & (c - 1) == 0
                    wgs = lambda ch: rows * -(-n // ch)
                    assert c == 64 or (c <= n and wgs(c) >= cus)
                    assert 2 * c > n or wgs(2 * c) < cus
    for args in ((0, 32, 8, 1000), (1, 0, 8, 1000), (1, 32, 0, 1000), (1, 32, 8, 0), (1, 30, 8, 1000)):
        with pytest.raises(ta.TreeAttnError) as e:
            ta.suggest_chunk(*args, compute_units=256)
        assert e.value.code == ta.TA_ERR_ARG


def test_merge_group_limit_is_refused_before_launch():
    # more leaves per row than 65535 workgroups of the first merge pass can take
    n = 65535 * 128 + 1
    po, pl = T([1, 1, n, 128], ta.TA_F32), T([1, 1, n], ta.TA_F32)
    out, lse = T([1, 1, 128], ta.TA_F32), T([1, 1], ta.TA_F32)
    rc, msg = call_combine(po, pl, n, out, lse)
    assert rc == ta.TA_ERR_UNSUPPORTED and "exceed" in msg
    assert call_combine(po, pl, n - 1, out, lse)[0] != ta.TA_ERR_UNSUPPORTED
    nk = 65535 * 512 + 1  # arity 8 takes 8^3 = 512 leaves per group
    pok, plk = T([1, 1, nk, 128], ta.TA_F32), T([1, 1, nk], ta.TA_F32)
    rc, msg = call_combine_k(pok, plk, nk, 8, out, lse)
    assert rc == ta.TA_ERR_UNSUPPORTED and "exceed" in msg
    assert call_combine_k(po, pl, n, 8, out, lse)[0] != ta.TA_ERR_UNSUPPORTED
    a = good(B=1, Hq=8, Hkv=8, N=n, d=128)  # chunk 1: one state per token
    rc, msg = call_decode(a, chunk=1)
    assert rc == ta.TA_ERR_UNSUPPORTED and "exceed" in msg


def test_lse_tensors_take_any_strides():
    # lse and partial_lse have no head dimension: non-unit and unaligned strides pass
    # validation (the calls then fail only for lack of a GPU, or succeed on one)
    po = T([2, 8, 16, 128], ta.TA_F32)
    pl = T([2, 8, 16], ta.TA_F32, stride=[1, 2, 16], data=FAKE + 4)
    out = T([2, 8, 128], ta.TA_F32)
    lse = T([2, 8], ta.TA_F32, stride=[3, 30], data=FAKE + 4)
    rc, msg = call_combine(po, pl, 16, out, lse)
    assert rc not in (ta.TA_ERR_STRIDE, ta.TA_ERR_SHAPE, ta.TA_ERR_DTYPE, ta.TA_ERR_ARG), msg
    bad = T([2, 8], ta.TA_F32, stride=[8, -1])
    assert call_combine(po, pl, 16, out, bad)[0] == ta.TA_ERR_STRIDE


def test_last_error_is_per_call():
    rc, msg = call_decode(good(), chunk=0)
    assert rc != 0 and msg
    rc, msg = call_decode(good(B=0))
    assert rc == 0 and msg == ""


def test_missing_library_fails_loudly(tmp_path):
    # no fallback: with the shared library absent, loading raises and names the build step
    import subprocess
    import sys
    code = (
        "import softmax_tree_reduction_amd as ta\n"
        f"ta._LIB_PATH = {str(tmp_path / 'libtreeattn.so')!r}\n"
        "try:\n"
        "    ta.load_library()\n"
        "except RuntimeError as e:\n"
        "    print('raised:', e)\n"
        "else:\n"
        "    print('loaded')\n"
    )
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120,
                       cwd=os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    assert "raised:" in r.stdout and "build" in r.stdout, r.stdout + r.stderr
