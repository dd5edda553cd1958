"""Python binding of libtreeattn.so: single-GPU Tree Attention decode on gfx950.

Argument marshalling only. Every step of the computation runs in the HIP
kernels behind the C ABI of include/tree_attn.h; torch supplies device memory
and streams. If the library is not built, every call raises: there is no
fallback path.

    out, lse = decode(q, k, v, seqlens=None, chunk=2048)
    po, pl   = partial(q, k, v, seqlens=None, chunk=2048)
    out, lse = combine(po, pl, n_parts=None)          # arity=k or "chain" for the other orders
    step = PreparedDecode(q, k, v, seqlens, chunk)    # fixed buffers: step() costs one C call
    chunk = suggest_chunk(B, Hq, Hkv, N)              # about one workgroup per compute unit
"""
from __future__ import annotations

import ctypes
import os
import threading

__all__ = ["decode", "decode_noalloc", "partial", "combine", "PreparedDecode", "stream_read", "suggest_chunk", "TreeAttnError",
           "library_path", "load_library",
           "TA_OK", "TA_ERR_NULL", "TA_ERR_SHAPE", "TA_ERR_DTYPE", "TA_ERR_STRIDE", "TA_ERR_ARG",
           "TA_ERR_UNSUPPORTED", "TA_ERR_HIP", "TaTensor", "EXPORTS"]

TA_OK, TA_ERR_NULL, TA_ERR_SHAPE, TA_ERR_DTYPE, TA_ERR_STRIDE, TA_ERR_ARG, TA_ERR_UNSUPPORTED, TA_ERR_HIP = \
    0, -1, -2, -3, -4, -5, -6, -7
TA_F32, TA_BF16 = 0, 1
EXPORTS = ("ta_decode", "ta_decode_noalloc", "ta_combine", "ta_combine_k", "ta_combine_chain", "ta_partial",
           "ta_stream_read", "ta_suggest_chunk", "ta_last_error", "ta_version")

_HERE = os.path.dirname(os.path.abspath(__file__))
# TA_LIBRARY names another build of the library to load (for instance the copy whose
# host code runs under sanitizers); by default the in-tree libtreeattn.so.
_LIB_PATH = os.environ.get("TA_LIBRARY") or os.path.join(_HERE, "libtreeattn.so")
_lock = threading.Lock()
_lib = None


class TreeAttnError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"tree_attn error {code}: {message}")
        self.code = code


class TaTensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("ndim", ctypes.c_int32),
                ("shape", ctypes.c_int64 * 4), ("stride", ctypes.c_int64 * 4)]

    @classmethod
    def make(cls, data: int, dtype: int, shape, stride) -> "TaTensor":
        t = cls()
        t.data = data
        t.dtype = dtype
        t.ndim = len(shape)
        for i, (s, st) in enumerate(zip(shape, stride)):
            t.shape[i] = int(s)
            t.stride[i] = int(st)
        return t


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libtreeattn.so (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH):
                raise RuntimeError(f"{_LIB_PATH} is missing: build it first (python -c 'import __graft_entry__ as g; g.build()')")
            lib = ctypes.CDLL(_LIB_PATH)
            P = ctypes.POINTER(TaTensor)
            vp, i32 = ctypes.c_void_p, ctypes.c_int32
            lib.ta_decode.argtypes = [P, P, P, vp, P, P, i32, vp]
            lib.ta_decode_noalloc.argtypes = [P, P, P, vp, P, P, i32, vp]
            lib.ta_partial.argtypes = [P, P, P, vp, P, P, i32, vp]
            lib.ta_combine.argtypes = [P, P, i32, P, P, vp]
            lib.ta_combine_k.argtypes = [P, P, i32, i32, P, P, vp]
            lib.ta_combine_chain.argtypes = [P, P, i32, P, P, vp]
            lib.ta_stream_read.argtypes = [vp, ctypes.c_int64, vp, vp]
            i64 = ctypes.c_int64
            lib.ta_suggest_chunk.argtypes = [i64, i64, i64, i64, i32]
            lib.ta_suggest_chunk.restype = ctypes.c_int32
            for f in (lib.ta_decode, lib.ta_decode_noalloc, lib.ta_partial, lib.ta_combine, lib.ta_combine_k, lib.ta_combine_chain,
                      lib.ta_stream_read):
                f.restype = ctypes.c_int
            lib.ta_last_error.restype = ctypes.c_char_p
            lib.ta_version.restype = ctypes.c_int
            _lib = lib
    return _lib


def _check(rc: int) -> None:
    if rc != TA_OK:
        msg = load_library().ta_last_error().decode(errors="replace")
        raise TreeAttnError(rc, msg)


# ----------------------------------------------------------------------------
# torch glue (imported lazily so the CPU-side ABI tests need no GPU). The calls
# below run once per decode step, so they keep the Python work per call small.
# ----------------------------------------------------------------------------

_DTYPES = None


def _dtype_code(t) -> int:
    global _DTYPES
    if _DTYPES is None:
        import torch
        _DTYPES = {torch.float32: TA_F32, torch.bfloat16: TA_BF16}
    dt = _DTYPES.get(t.dtype)
    if dt is None:
        raise TypeError(f"unsupported dtype {t.dtype}: use float32 or bfloat16")
    return dt


def _desc(t) -> TaTensor:
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    d = TaTensor()
    d.data = t.data_ptr()
    d.dtype = _dtype_code(t)
    shape, stride = t.shape, t.stride()
    n = len(shape)
    d.ndim = n
    d.shape[0:n] = shape
    d.stride[0:n] = stride
    return d


def _call(dev, stream, fn):
    """Run fn(stream_handle) with `dev` current."""
    import torch
    if torch.cuda.current_device() != dev.index:
        with torch.cuda.device(dev):
            return _call(dev, stream, fn)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    _check(fn(ctypes.c_void_p(stream.cuda_stream)))


def _seqlens_ptr(seqlens, B, device):
    import torch
    if seqlens is None:
        return None
    if not (seqlens.is_cuda and seqlens.dtype == torch.int32 and seqlens.is_contiguous() and seqlens.numel() == B):
        raise ValueError("seqlens must be a contiguous int32 CUDA tensor with one entry per sequence")
    if seqlens.device != device:
        raise ValueError("seqlens must be on the same device as q")
    return ctypes.c_void_p(seqlens.data_ptr())


def _same_device(*ts):
    dev = ts[0].device
    for t in ts[1:]:
        if t is not None and t.device != dev:
            raise ValueError("all tensors must be on the same device")
    return dev


def decode(q, k, v, seqlens=None, chunk: int = 2048, out=None, lse=None, stream=None):
    """One decode step: returns (out [B, Hq, d] f32, lse [B, Hq] f32)."""
    import torch
    dev = _same_device(q, k, v, out, lse)
    B, Hq, d = q.shape
    if out is None:
        out = torch.empty(B, Hq, d, dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty(B, Hq, dtype=torch.float32, device=dev)
    sl = _seqlens_ptr(seqlens, B, dev)
    lib = _lib or load_library()
    dq, dk, dv, do, dl = _desc(q), _desc(k), _desc(v), _desc(out), _desc(lse)
    by = ctypes.byref
    _call(dev, stream, lambda s: lib.ta_decode(by(dq), by(dk), by(dv), sl, by(do), by(dl), int(chunk), s))
    return out, lse


def decode_noalloc(q, k, v, seqlens=None, chunk: int = 2048, out=None, lse=None, stream=None):
    """ta_decode_noalloc: decode() whose partial states live in the library's static
    device scratch (64 MiB per device) instead of allocated workspace. The library
    allocates nothing; out and lse are allocated here only when not given. Calls
    whose work overlaps on one device (different unordered streams) race."""
    import torch
    dev = _same_device(q, k, v, out, lse)
    B, Hq, d = q.shape
    if out is None:
        out = torch.empty(B, Hq, d, dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty(B, Hq, dtype=torch.float32, device=dev)
    sl = _seqlens_ptr(seqlens, B, dev)
    lib = _lib or load_library()
    dq, dk, dv, do, dl = _desc(q), _desc(k), _desc(v), _desc(out), _desc(lse)
    by = ctypes.byref
    _call(dev, stream, lambda s: lib.ta_decode_noalloc(by(dq), by(dk), by(dv), sl, by(do), by(dl), int(chunk), s))
    return out, lse


class PreparedDecode:
    """ta_decode on fixed buffers, for loops that call it many times.

    The descriptors of q, k, v, out and lse are built once; each call then costs
    one C call. The buffers are read when the call runs, so the caller refills q,
    k, v and seqlens in place between calls and reads out and lse after them.
    The tensors must stay alive and keep their storage while the object is used.
    """

    def __init__(self, q, k, v, seqlens=None, chunk: int = 2048, out=None, lse=None):
        import torch
        dev = _same_device(q, k, v, out, lse)
        B, Hq, d = q.shape
        self.out = out if out is not None else torch.empty(B, Hq, d, dtype=torch.float32, device=dev)
        self.lse = lse if lse is not None else torch.empty(B, Hq, dtype=torch.float32, device=dev)
        self._keep = (q, k, v, seqlens)
        self._dev = dev
        self._sl = _seqlens_ptr(seqlens, B, dev)
        self._chunk = int(chunk)
        self._d = [_desc(q), _desc(k), _desc(v), _desc(self.out), _desc(self.lse)]
        self._lib = _lib or load_library()

    def __call__(self, stream=None):
        """Enqueues one decode step on `stream` (torch's current stream by default)."""
        by = ctypes.byref
        dq, dk, dv, do, dl = self._d
        _call(self._dev, stream,
              lambda s: self._lib.ta_decode(by(dq), by(dk), by(dv), self._sl, by(do), by(dl), self._chunk, s))
        return self.out, self.lse


def partial(q, k, v, seqlens=None, chunk: int = 2048, partial_o=None, partial_lse=None, stream=None):
    """Per-chunk partial states: returns (partial_o [B, Hq, P, d], partial_lse [B, Hq, P]), f32."""
    import torch
    dev = _same_device(q, k, v, partial_o, partial_lse)
    B, Hq, d = q.shape
    N = k.shape[2]
    P = max(1, -(-N // int(chunk))) if chunk > 0 else 1
    if partial_o is None:
        partial_o = torch.empty(B, Hq, P, d, dtype=torch.float32, device=dev)
    if partial_lse is None:
        partial_lse = torch.empty(B, Hq, P, dtype=torch.float32, device=dev)
    sl = _seqlens_ptr(seqlens, B, dev)
    lib = _lib or load_library()
    dq, dk, dv, dpo, dpl = _desc(q), _desc(k), _desc(v), _desc(partial_o), _desc(partial_lse)
    by = ctypes.byref
    _call(dev, stream, lambda s: lib.ta_partial(by(dq), by(dk), by(dv), sl, by(dpo), by(dpl), int(chunk), s))
    return partial_o, partial_lse


def combine(partial_o, partial_lse, n_parts=None, out=None, lse=None, stream=None, arity=None):
    """Tree merge of partial states: returns (out [B, H, d] f32, lse [B, H] f32).

    arity None runs ta_combine (the binary tree); an integer in [2, 16] runs
    ta_combine_k with that branching factor; "chain" runs ta_combine_chain, the
    sequential order of a ring.
    """
    import torch
    dev = _same_device(partial_o, partial_lse, out, lse)
    B, H, P, d = partial_o.shape
    if n_parts is None:
        n_parts = P
    if out is None:
        out = torch.empty(B, H, d, dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty(B, H, dtype=torch.float32, device=dev)
    lib = _lib or load_library()
    dpo, dpl, do, dl = _desc(partial_o), _desc(partial_lse), _desc(out), _desc(lse)
    by = ctypes.byref
    if arity is None:
        _call(dev, stream, lambda s: lib.ta_combine(by(dpo), by(dpl), int(n_parts), by(do), by(dl), s))
    elif arity == "chain":
        _call(dev, stream, lambda s: lib.ta_combine_chain(by(dpo), by(dpl), int(n_parts), by(do), by(dl), s))
    else:
        _call(dev, stream, lambda s: lib.ta_combine_k(by(dpo), by(dpl), int(n_parts), int(arity), by(do), by(dl), s))
    return out, lse


def stream_read(buf, sink, stream=None):
    """Read-bandwidth probe (ta_stream_read): streams every byte of the CUDA tensor
    `buf` once; `sink` is a CUDA tensor of at least 4 bytes the probe may write."""
    dev = _same_device(buf, sink)
    if not (buf.is_cuda and sink.is_cuda and buf.is_contiguous() and sink.numel() * sink.element_size() >= 4):
        raise ValueError("buf must be a contiguous CUDA tensor and sink a CUDA tensor of >= 4 bytes")
    lib = _lib or load_library()
    nbytes = buf.numel() * buf.element_size()
    _call(dev, stream, lambda s: lib.ta_stream_read(ctypes.c_void_p(buf.data_ptr()), ctypes.c_int64(nbytes),
                                                    ctypes.c_void_p(sink.data_ptr()), s))


def suggest_chunk(batch: int, q_heads: int, kv_heads: int, n: int, compute_units: int = 0) -> int:
    """ta_suggest_chunk: the largest power-of-two chunk (>= 64, <= n) that still gives
    the partial kernel at least one workgroup per compute unit; compute_units 0 asks
    the current device. Meant for batches whose sequences all hold n tokens."""
    lib = _lib or load_library()
    c = lib.ta_suggest_chunk(int(batch), int(q_heads), int(kv_heads), int(n), int(compute_units))
    _check(c if c < 0 else TA_OK)
    return int(c)
