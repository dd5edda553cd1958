"""Shared pieces of the GPU parity tests: moving generator output to the device
and the tolerances every comparison uses.

Tolerances: max |out - oracle| <= 1e-5 for float32 inputs and <= 4e-3 for
bfloat16 inputs; |lse - oracle| <= 1e-4 * max(1, |oracle lse|), a relative bound
with an absolute floor for the few tiny cases whose lse is near 0 (every
workload-sized case has lse well above 1); where the oracle's lse is -inf (no tokens) the GPU's must be -inf too and its output exactly 0.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

OUT_TOL = {"f32": 1e-5, "bf16": 4e-3}
LSE_RTOL = 1e-4


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def dev_tensor(a: np.ndarray, device="cuda") -> torch.Tensor:
    """float32 arrays as float32; uint16 arrays (bfloat16 bits) as bfloat16."""
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def upload(inp, device="cuda"):
    q = dev_tensor(inp.q, device)
    k = dev_tensor(inp.k, device)
    v = dev_tensor(inp.v, device)
    sl = torch.from_numpy(np.asarray(inp.seqlens, dtype=np.int32)).to(device)
    return q, k, v, sl


def assert_close(out, lse, ref_out, ref_lse, dtype: str, what: str = ""):
    """out/lse: numpy arrays from the GPU; ref_*: float64 oracle arrays of the same shape."""
    out = np.asarray(out, dtype=np.float64)
    lse = np.asarray(lse, dtype=np.float64)
    empty = np.isneginf(ref_lse)
    assert np.array_equal(np.isneginf(lse), empty), f"{what}: empty rows differ"
    if empty.any():
        assert np.all(out[empty] == 0.0), f"{what}: empty rows must be 0"
    full = ~empty
    if full.any():
        err = np.abs(out[full] - ref_out[full]).max()
        assert np.isfinite(out[full]).all(), f"{what}: non-finite output"
        assert err <= OUT_TOL[dtype], f"{what}: max |out - oracle| = {err:.3e} > {OUT_TOL[dtype]}"
        lerr = (np.abs(lse[full] - ref_lse[full]) / np.maximum(1.0, np.abs(ref_lse[full]))).max()
        assert lerr <= LSE_RTOL, f"{what}: max rel lse error {lerr:.3e} > {LSE_RTOL}"
        return err, lerr
    return 0.0, 0.0
