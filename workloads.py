"""Seeded synthetic inputs for single-query decode attention over a KV cache.

This module only draws numbers. It holds none of the attention arithmetic, so
both the HIP path and the CPU oracle can take their inputs from it without
sharing any of the method's code.

Recipe (every draw is reproducible from the seed, independent of thread count):

* Every tensor is filled block by block. Block ``i`` of tensor ``t`` draws from
  its own ``numpy.random.PCG64`` stream seeded by
  ``SeedSequence(seed, spawn_key=(t, i))``, so blocks can be drawn by a thread
  pool in any order. A block is ``2**22`` values in the tensor's row-major order.
* Values are standard normal float32. For bf16 tensors each float32 is rounded
  to the nearest bfloat16, ties to even (the bf16 format is the top 16 bits of
  the float32 one); the generator never produces NaN or Inf, so no NaN case is
  needed in the rounding.
* Tensor ids: 0 = ragged lengths, 1 = q, 2 = K, 3 = V, 4 = the peaked-key row
  mask, 5 = combine partial outputs, 6 = combine partial log-sum-exps.
* The peaked-key workload selects each K row (batch, kv head, token)
  independently with probability 0.01 and multiplies the whole row by 8 before
  rounding (a power of two, so rounding commutes with it).
* Ragged workloads draw integer lengths uniform on [lo, hi] inclusive; rows past
  a sequence's length are filled with NaN so that any read past the end
  poisons the result instead of passing silently.
* q is drawn N(0,1) unscaled; the 1/sqrt(d) attention scale is applied by the
  attention itself.

Arrays are returned as numpy arrays in host memory: float32, or uint16 holding
bfloat16 bit patterns.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

BLOCK = 1 << 22
TENSOR_LENS, TENSOR_Q, TENSOR_K, TENSOR_V, TENSOR_MASK, TENSOR_PO, TENSOR_PLSE = range(7)
BF16_NAN = np.uint16(0x7FC0)


def _threads() -> int:
    env = os.environ.get("WORKLOADS_THREADS")
    if env:
        return max(1, int(env))
    return max(1, min(16, os.cpu_count() or 1))


def _stream(seed: int, tensor: int, block: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(tensor, block))))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); returns uint16 bits.

    Finite inputs only. The rounding adds 0x7FFF plus the lowest kept bit to
    the 32-bit pattern and keeps the top half, which rounds the dropped 16
    bits to nearest with ties going to the even kept value.
    """
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).copy()
    b += np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))
    return (b >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32 (for reports and tests)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal(seed: int, tensor: int, n: int, *, mean: float = 0.0, std: float = 1.0) -> np.ndarray:
    """n float32 values N(mean, std^2), drawn block-parallel from the tensor's streams."""
    out = np.empty(n, dtype=np.float32)
    nblk = (n + BLOCK - 1) // BLOCK

    def fill(i: int) -> None:
        lo, hi = i * BLOCK, min(n, (i + 1) * BLOCK)
        _stream(seed, tensor, i).standard_normal(out=out[lo:hi], dtype=np.float32)
        if std != 1.0 or mean != 0.0:
            out[lo:hi] *= np.float32(std)
            out[lo:hi] += np.float32(mean)

    if nblk <= 1:
        for i in range(nblk):
            fill(i)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nblk)))
    return out


def uniform01(seed: int, tensor: int, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.float64)
    nblk = (n + BLOCK - 1) // BLOCK
    for i in range(nblk):
        lo, hi = i * BLOCK, min(n, (i + 1) * BLOCK)
        out[lo:hi] = _stream(seed, tensor, i).random(hi - lo)
    return out


def _to_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return x
    if dtype == "bf16":
        # convert in slices so the uint32 temporary stays small
        out = np.empty(x.shape, dtype=np.uint16)
        flat_in, flat_out = x.reshape(-1), out.reshape(-1)
        step = 1 << 24

        def conv(i: int) -> None:
            flat_out[i:i + step] = f32_to_bf16_bits(flat_in[i:i + step])

        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(conv, range(0, flat_in.size, step)))
        return out
    raise ValueError(f"unknown dtype {dtype!r}")


@dataclass(frozen=True)
class DecodeWorkload:
    """Shape of one decode step: batch B, Hq query heads sharing Hkv KV heads, head dim d."""
    name: str
    B: int
    Hq: int
    Hkv: int
    d: int
    N: int                       # cache capacity per sequence (padded length for ragged batches)
    chunk: int                   # tokens per partial state
    dtype: str                   # "f32" or "bf16" for q, K and V
    ragged: tuple | None = None  # (lo, hi) inclusive range of sequence lengths
    spike_frac: float = 0.0      # fraction of K rows scaled by spike_scale
    spike_scale: float = 8.0
    description: str = ""


@dataclass(frozen=True)
class CombineWorkload:
    name: str
    B: int
    H: int
    n_parts: int
    d: int
    lse_mean: float = 10.0
    lse_std: float = 3.0
    description: str = ""


# The workloads: a tiny fp32 case, then Llama-3.1-8B attention shapes
# (32 query heads, 8 KV heads, head dim 128) at long contexts.
WORKLOADS = {
    "tiny_f32": DecodeWorkload(
        "tiny_f32", B=1, Hq=1, Hkv=1, d=64, N=4096, chunk=512, dtype="f32",
        description="1 head, d=64, 4096 keys, fp32, 8 chunks of 512"),
    "gqa8b_128k": DecodeWorkload(
        "gqa8b_128k", B=1, Hq=32, Hkv=8, d=128, N=131072, chunk=2048, dtype="bf16",
        description="Llama-3.1-8B GQA 32/8, d=128, bf16, 128k context, chunk 2048 (64 partials)"),
    "gqa8b_512k_b4_peaked": DecodeWorkload(
        "gqa8b_512k_b4_peaked", B=4, Hq=32, Hkv=8, d=128, N=524288, chunk=4096, dtype="bf16",
        spike_frac=0.01, spike_scale=8.0,
        description="8B GQA, bf16, batch 4 x 512k, chunk 4096, 1% of K rows x8"),
    "gqa8b_1m": DecodeWorkload(
        "gqa8b_1m", B=1, Hq=32, Hkv=8, d=128, N=1048576, chunk=8192, dtype="bf16",
        description="8B GQA, bf16, one 1M-token sequence, chunk 8192 (128 partials)"),
    "gqa8b_ragged_b32": DecodeWorkload(
        "gqa8b_ragged_b32", B=32, Hq=32, Hkv=8, d=128, N=65536, chunk=1024, dtype="bf16",
        ragged=(4096, 65536),
        description="8B GQA, bf16, batch 32, lengths uniform in [4096, 65536], chunk 1024"),
}

COMBINE_WORKLOADS = {
    "combine_64x128": CombineWorkload(
        "combine_64x128", B=32, H=32, n_parts=64, d=128,
        description="merge 64 fp32 (o[128], lse) partial states per head, 32 x 32 heads"),
}


@dataclass
class DecodeInputs:
    wl: DecodeWorkload
    seed: int
    q: np.ndarray         # [B, Hq, d]
    k: np.ndarray         # [B, Hkv, N, d]
    v: np.ndarray         # [B, Hkv, N, d]
    seqlens: np.ndarray   # int32 [B]
    meta: dict = field(default_factory=dict)


def seqlens_for(wl: DecodeWorkload, seed: int) -> np.ndarray:
    if wl.ragged is None:
        return np.full(wl.B, wl.N, dtype=np.int32)
    lo, hi = wl.ragged
    g = _stream(seed, TENSOR_LENS, 0)
    return g.integers(lo, hi, size=wl.B, endpoint=True).astype(np.int32)


def make_decode_inputs(wl: DecodeWorkload, seed: int) -> DecodeInputs:
    """Draw q, K, V and the sequence lengths of one decode step."""
    B, Hq, Hkv, N, d = wl.B, wl.Hq, wl.Hkv, wl.N, wl.d
    seqlens = seqlens_for(wl, seed)
    q = _to_dtype(normal(seed, TENSOR_Q, B * Hq * d).reshape(B, Hq, d), wl.dtype)

    def cache(tensor: int) -> np.ndarray:
        if wl.ragged is None:
            x = normal(seed, tensor, B * Hkv * N * d).reshape(B, Hkv, N, d)
            if tensor == TENSOR_K and wl.spike_frac > 0:
                u = uniform01(seed, TENSOR_MASK, B * Hkv * N).reshape(B, Hkv, N)
                x[u < wl.spike_frac] *= np.float32(wl.spike_scale)
            return _to_dtype(x, wl.dtype)
        # ragged: draw only the valid rows (sequence by sequence, head by head, in
        # that order), NaN past each sequence's end
        total = int(seqlens.sum()) * Hkv * d
        flat = _to_dtype(normal(seed, tensor, total), wl.dtype)
        out = np.empty((B, Hkv, N, d), dtype=flat.dtype)
        nan = BF16_NAN if wl.dtype == "bf16" else np.float32(np.nan)
        off = 0
        for b in range(B):
            n = int(seqlens[b])
            for h in range(Hkv):
                out[b, h, :n] = flat[off:off + n * d].reshape(n, d)
                out[b, h, n:] = nan
                off += n * d
        return out

    k = cache(TENSOR_K)
    v = cache(TENSOR_V)
    return DecodeInputs(wl, seed, q, k, v, seqlens, meta={"numpy": np.__version__})


@dataclass
class CombineInputs:
    wl: CombineWorkload
    seed: int
    partial_o: np.ndarray    # float32 [B, H, n_parts, d]
    partial_lse: np.ndarray  # float32 [B, H, n_parts]


def make_combine_inputs(wl: CombineWorkload, seed: int) -> CombineInputs:
    B, H, P, d = wl.B, wl.H, wl.n_parts, wl.d
    po = normal(seed, TENSOR_PO, B * H * P * d).reshape(B, H, P, d)
    pl = normal(seed, TENSOR_PLSE, B * H * P, mean=wl.lse_mean, std=wl.lse_std).reshape(B, H, P)
    return CombineInputs(wl, seed, po, pl)


def random_decode(B: int, Hq: int, Hkv: int, N: int, d: int, dtype: str, seed: int,
                  seqlens=None, spike_frac: float = 0.0, chunk: int = 256,
                  name: str = "custom") -> DecodeInputs:
    """A small workload of any shape (tests)."""
    ragged = None
    wl = DecodeWorkload(name, B=B, Hq=Hq, Hkv=Hkv, d=d, N=N, chunk=chunk, dtype=dtype,
                        ragged=ragged, spike_frac=spike_frac)
    inp = make_decode_inputs(wl, seed)
    if seqlens is not None:
        sl = np.asarray(seqlens, dtype=np.int32)
        assert sl.shape == (B,) and (sl >= 0).all() and (sl <= N).all()
        nan = BF16_NAN if dtype == "bf16" else np.float32(np.nan)
        for b in range(B):
            inp.k[b, :, sl[b]:] = nan
            inp.v[b, :, sl[b]:] = nan
        inp.seqlens = sl
    return inp
