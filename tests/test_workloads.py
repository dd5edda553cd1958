"""The seeded input generator: reproducible, thread-count independent, and
shaped like the workloads it stands in for."""
from __future__ import annotations

import numpy as np

import workloads as W


def test_same_seed_same_inputs_any_thread_count(monkeypatch):
    wl = W.DecodeWorkload("t", B=2, Hq=4, Hkv=2, d=64, N=1 << 15, chunk=512, dtype="bf16")
    monkeypatch.setenv("WORKLOADS_THREADS", "1")
    a = W.make_decode_inputs(wl, 3)
    monkeypatch.setenv("WORKLOADS_THREADS", "7")
    b = W.make_decode_inputs(wl, 3)
    for x, y in [(a.q, b.q), (a.k, b.k), (a.v, b.v), (a.seqlens, b.seqlens)]:
        assert np.array_equal(x, y)
    c = W.make_decode_inputs(wl, 4)
    assert not np.array_equal(a.k, c.k)


def test_ragged_lengths_and_nan_tail():
    wl = W.DecodeWorkload("r", B=6, Hq=4, Hkv=2, d=16, N=512, chunk=64, dtype="bf16", ragged=(10, 500))
    inp = W.make_decode_inputs(wl, 1)
    assert inp.seqlens.dtype == np.int32
    assert (inp.seqlens >= 10).all() and (inp.seqlens <= 500).all()
    for b in range(6):
        n = inp.seqlens[b]
        tail = W.bf16_bits_to_f32(inp.k[b, :, n:])
        head = W.bf16_bits_to_f32(inp.k[b, :, :n])
        assert np.isnan(tail).all() and np.isfinite(head).all()


def test_peaked_keys_fraction_and_scale():
    wl = W.DecodeWorkload("p", B=1, Hq=4, Hkv=2, d=32, N=1 << 16, chunk=512, dtype="f32",
                          spike_frac=0.01, spike_scale=8.0)
    inp = W.make_decode_inputs(wl, 2)
    base = W.DecodeWorkload("p0", B=1, Hq=4, Hkv=2, d=32, N=1 << 16, chunk=512, dtype="f32")
    ref = W.make_decode_inputs(base, 2)
    scaled = np.all(inp.k == np.float32(8.0) * ref.k, axis=-1)
    unscaled = np.all(inp.k == ref.k, axis=-1)
    assert np.all(scaled | unscaled)
    frac = scaled.mean()
    assert 0.008 < frac < 0.012
    assert np.array_equal(inp.v, ref.v)


def test_standard_normal_moments():
    x = W.normal(5, W.TENSOR_K, 1 << 20)
    assert abs(x.mean()) < 5e-3 and abs(x.std() - 1) < 5e-3


def test_combine_inputs_shape():
    wl = W.CombineWorkload("c", B=2, H=3, n_parts=5, d=8)
    ci = W.make_combine_inputs(wl, 1)
    assert ci.partial_o.shape == (2, 3, 5, 8) and ci.partial_lse.shape == (2, 3, 5)
    assert abs(ci.partial_lse.mean() - 10) < 3
