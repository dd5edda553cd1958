"""ta_decode_noalloc, the allocation-free decode: its partial states and merge
scratch live in the library's static device array. It runs the kernels of
ta_decode, so its results must equal ta_decode's bit for bit; they are also
checked against the float64 oracle. The array keeps the last call's contents,
so calls follow each other with different (and smaller) inputs."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

import oracle
import softmax_tree_reduction_amd as ta
import workloads as W
from gpu_helpers import assert_close, log, upload

FAKE = 0x10000  # validation never reads it


def _T(shape, dtype, data=FAKE):
    stride, acc = [], 1
    for s in reversed(shape):
        stride.insert(0, acc)
        acc *= s
    return ta.TaTensor.make(data, dtype, shape, stride)


def test_noalloc_refuses_a_step_beyond_its_scratch():
    # 64 sequences x 64 heads x 1024 states x 129 floats: about 2.2 GB of partial
    # states, refused before any device call (the pointers are never read)
    lib = ta.load_library()
    B, Hq, Hkv, N, d = 64, 64, 8, 1 << 20, 128
    q, k, v = _T([B, Hq, d], ta.TA_BF16), _T([B, Hkv, N, d], ta.TA_BF16), _T([B, Hkv, N, d], ta.TA_BF16)
    out, lse = _T([B, Hq, d], ta.TA_F32), _T([B, Hq], ta.TA_F32)
    by = ctypes.byref
    rc = lib.ta_decode_noalloc(by(q), by(k), by(v), None, by(out), by(lse), 1024, None)
    msg = lib.ta_last_error().decode()
    assert rc == ta.TA_ERR_UNSUPPORTED, msg
    assert "static scratch" in msg and "67108864" in msg
    # validation failures come first, as for ta_decode
    rc = lib.ta_decode_noalloc(by(q), by(k), by(v), None, by(out), by(lse), 0, None)
    assert rc == ta.TA_ERR_ARG


def _case(B, Hq, Hkv, N, d, dtype, seed, seqlens, chunk):
    inp = W.random_decode(B=B, Hq=Hq, Hkv=Hkv, N=N, d=d, dtype=dtype, seed=seed, seqlens=seqlens)
    return inp, chunk


@pytest.mark.gpu
def test_noalloc_equals_decode_on_calls_in_a_row():
    cases = [
        # large first: a ragged GQA batch; then smaller ones that leave stale states
        # of the first behind them in the array
        _case(4, 32, 8, 40000, 128, "bf16", 71, [40000, 123, 39999, 0], 512),
        _case(2, 8, 2, 3000, 128, "bf16", 72, [3000, 1777], 256),
        # more than 128 states per row: the merge runs in passes through the array too
        _case(2, 8, 2, 20000, 128, "bf16", 73, [20000, 9001], 64),
        _case(1, 4, 4, 5000, 64, "f32", 74, [4321], 37),
    ]
    for i, (inp, chunk) in enumerate(cases):
        q, k, v, sl = upload(inp)
        log(f"noalloc call {i}: B={inp.q.shape[0]} Hq={inp.q.shape[1]} Hkv={inp.k.shape[1]} N={inp.k.shape[2]} "
            f"d={inp.q.shape[2]} chunk={chunk}")
        o_na, l_na = ta.decode_noalloc(q, k, v, sl, chunk=chunk)
        o_ref, l_ref = ta.decode(q, k, v, sl, chunk=chunk)
        torch.cuda.synchronize()
        assert torch.equal(o_na, o_ref) and torch.equal(l_na, l_ref), f"call {i}: differs from ta_decode"
        ro, rl = oracle.decode(inp.q, inp.k, inp.v, inp.seqlens)
        dtype = "bf16" if inp.q.dtype == np.uint16 else "f32"
        assert_close(o_na.cpu().numpy(), l_na.cpu().numpy(), ro, rl, dtype, what=f"noalloc call {i}")


@pytest.mark.gpu
def test_noalloc_full_size_128k_step():
    # the benchmark's 128k workload (1.06 MB of states): equal to ta_decode bit for bit
    wl = W.WORKLOADS["gqa8b_128k"]
    inp = W.make_decode_inputs(wl, 1)
    q, k, v, _ = upload(inp)
    log("noalloc: 128k workload")
    o_na, l_na = ta.decode_noalloc(q, k, v, None, chunk=wl.chunk)
    o_ref, l_ref = ta.decode(q, k, v, None, chunk=wl.chunk)
    torch.cuda.synchronize()
    assert torch.equal(o_na, o_ref) and torch.equal(l_na, l_ref)


@pytest.mark.gpu
def test_noalloc_graph_replays_match_eager():
    inp = W.random_decode(B=2, Hq=8, Hkv=2, N=5000, d=128, dtype="bf16", seed=75, seqlens=[5000, 2222])
    other = W.random_decode(B=1, Hq=8, Hkv=2, N=3000, d=128, dtype="bf16", seed=76, seqlens=[2500])
    q, k, v, sl = upload(inp)
    q2, k2, v2, sl2 = upload(other)
    ref_o, ref_l = ta.decode(q, k, v, sl, chunk=256)
    ref2_o, ref2_l = ta.decode(q2, k2, v2, sl2, chunk=128)
    out = torch.empty_like(ref_o)
    lse = torch.empty_like(ref_l)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        ta.decode_noalloc(q, k, v, sl, chunk=256, out=out, lse=lse)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    log("noalloc: capturing")
    with torch.cuda.graph(g):
        ta.decode_noalloc(q, k, v, sl, chunk=256, out=out, lse=lse)
    for rep in range(3):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), f"replay {rep}"
        # an eager allocation-free call with another shape between replays overwrites the array
        o2, l2 = ta.decode_noalloc(q2, k2, v2, sl2, chunk=128)
        torch.cuda.synchronize()
        assert torch.equal(o2, ref2_o) and torch.equal(l2, ref2_l)
    del g
    torch.cuda.synchronize()
