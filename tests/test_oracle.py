"""Pins of the CPU oracle against things other than itself.

The oracle (``oracle/``) is the plain float64 definition of single-query
attention, softmax(q K^T / sqrt(d)) V with its log-sum-exp, plus the page's
merge operator and tree fold. Each test below ties it to an independent fact:

* brute force at 50 significant digits, written in a different form (no max
  shift, weights exp(s_j) / sum_i exp(s_i), GQA spelled out head by head);
* a library routine: torch's scaled_dot_product_attention and logsumexp in
  float64 on the CPU;
* closed forms (constant keys, one dominant key, one token, constant values,
  shifted values) and bounds;
* the associativity claim of "Tree Attention Guide: Topology-Aware LLM
  Decoding", section "Core Innovation 2: Mathematical Formulation of Online
  Softmax on Trees" (any chunking and any tree shape give the unchunked
  result), enumerated exhaustively on small inputs;
* the tree depths printed in section "Core Innovation 1" step 3 of the same
  page (tests/golden/tree_depths.json).

Each is chosen so that a plausible slip in the oracle (a dropped scale, a
wrong GQA index, a transposed operand, a sign, a missing term) fails at least
one of them; ``test_planted_mistakes_are_caught`` checks exactly that on
mutated copies of the oracle source.
"""
from __future__ import annotations

import itertools
import json
import math
import os
import subprocess
import ctypes

import mpmath
import numpy as np
import pytest
import torch

import oracle
import workloads as W

HERE = os.path.dirname(os.path.abspath(__file__))


# --------------------------------------------------------------------------
# helpers that do not use the oracle
# --------------------------------------------------------------------------

def widen(x: np.ndarray) -> np.ndarray:
    """Stored values as float64 (bf16 bits widen exactly)."""
    if x.dtype == np.uint16:
        return W.bf16_bits_to_f32(x).astype(np.float64)
    return x.astype(np.float64)


def brute_force(q, k, v, seqlens, dps: int = 50):
    """Definition at `dps` digits: w_j = exp(s_j) / sum_i exp(s_i), no max shift."""
    mpmath.mp.dps = dps
    qf, kf, vf = widen(q), widen(k), widen(v)
    B, Hq, d = qf.shape
    Hkv = kf.shape[1]
    G = Hq // Hkv
    out = np.zeros((B, Hq, d))
    lse = np.zeros((B, Hq))
    inv_sqrt_d = 1 / mpmath.sqrt(d)
    for b in range(B):
        n = int(seqlens[b])
        for h in range(Hq):
            kv = h // G  # query heads G*g .. G*g+G-1 read KV head g
            if n == 0:
                lse[b, h] = -math.inf
                continue
            e = []
            for j in range(n):
                s = mpmath.fsum(mpmath.mpf(qf[b, h, c]) * mpmath.mpf(kf[b, kv, j, c]) for c in range(d))
                e.append(mpmath.exp(s * inv_sqrt_d))
            z = mpmath.fsum(e)
            lse[b, h] = float(mpmath.log(z))
            for c in range(d):
                out[b, h, c] = float(mpmath.fsum(e[j] * mpmath.mpf(vf[b, kv, j, c]) for j in range(n)) / z)
    return out, lse


def window_state(q, k, v, seqlens, t0, t1):
    """The oracle restricted to tokens [t0, t1), as a normalised state per row."""
    return oracle.decode(q, k, v, seqlens, t_begin=t0, t_end=t1)


def compositions(n):
    """All ways to cut range(n) into consecutive non-empty chunks: lists of (t0, t1)."""
    for cuts in itertools.product([0, 1], repeat=n - 1):
        bounds, start = [], 0
        for i, c in enumerate(cuts, start=1):
            if c:
                bounds.append((start, i))
                start = i
        bounds.append((start, n))
        yield bounds


def all_trees(states):
    """Every full binary tree over the ordered leaves, folded with the merge operator."""
    if len(states) == 1:
        yield states[0]
        return
    for split in range(1, len(states)):
        for left in all_trees(states[:split]):
            for right in all_trees(states[split:]):
                yield oracle.merge(left, right)


# --------------------------------------------------------------------------
# the bf16 rounding of the input generator (a library routine pins it)
# --------------------------------------------------------------------------

def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(100000).astype(np.float32) * np.float32(10.0) ** rng.integers(-30, 30, 100000).astype(np.float32),
        # exact ties: low 16 bits 0x8000, both parities of the kept bit
        (np.arange(1000, dtype=np.uint32) << 16 | 0x8000).view(np.float32),
        np.array([0.0, -0.0, 1.0, -1.0, 3.0e38, -3.0e38, 1e-40, -1e-40], dtype=np.float32),
    ]).astype(np.float32)
    x = x[np.isfinite(x)]
    ours = W.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = W.bf16_bits_to_f32(ours)
    assert np.array_equal(torch.from_numpy(back).numpy(), torch.from_numpy(ours.view(np.int16)).view(torch.bfloat16).float().numpy())


# --------------------------------------------------------------------------
# P1: brute force on tiny inputs (GQA, ragged, both dtypes)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("seed", [1, 2])
def test_brute_force_tiny(dtype, seed):
    inp = W.random_decode(B=2, Hq=4, Hkv=2, N=7, d=3, dtype=dtype, seed=seed, seqlens=[7, 4])
    out, lse = oracle.decode(inp.q, inp.k, inp.v, inp.seqlens)
    bo, bl = brute_force(inp.q, inp.k, inp.v, inp.seqlens)
    np.testing.assert_allclose(out, bo, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse, bl, rtol=1e-13, atol=1e-14)


def test_brute_force_head_dim_and_gqa_ratio():
    # d = 5 (odd), G = 3, one query head per KV head in the second case
    for (Hq, Hkv, d) in [(6, 2, 5), (3, 3, 4)]:
        inp = W.random_decode(B=1, Hq=Hq, Hkv=Hkv, N=6, d=d, dtype="f32", seed=11, seqlens=[6])
        out, lse = oracle.decode(inp.q, inp.k, inp.v, inp.seqlens)
        bo, bl = brute_force(inp.q, inp.k, inp.v, inp.seqlens)
        np.testing.assert_allclose(out, bo, rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(lse, bl, rtol=1e-13, atol=1e-14)


def test_selected_rows_match_full():
    inp = W.random_decode(B=3, Hq=8, Hkv=2, N=50, d=16, dtype="bf16", seed=5, seqlens=[50, 17, 1])
    out, lse = oracle.decode(inp.q, inp.k, inp.v, inp.seqlens)
    rows = np.array([23, 0, 9, 15, 16, 8])
    so, sl = oracle.decode(inp.q, inp.k, inp.v, inp.seqlens, rows=rows)
    np.testing.assert_array_equal(so, out.reshape(-1, 16)[rows])
    np.testing.assert_array_equal(sl, lse.reshape(-1)[rows])


# --------------------------------------------------------------------------
# P2: a small worked example with a known answer
# --------------------------------------------------------------------------

def test_worked_example_weights_quarter_three_quarters():
    # d = 1, q = 1: logits 0 and ln 3, softmax weights 1/4 and 3/4 over values 4 and 8:
    # out = 7 and lse = ln(1 + 3) = ln 4. ln 3 is rounded to float32 (|err| < 6e-8), which
    # moves out by at most (dout/ds) * err = 4 * 3/16 * 6e-8 < 5e-8 and lse by 3/4 * err.
    q = np.array([[[1.0]]], dtype=np.float32)
    k = np.array([[[[0.0], [math.log(3.0)]]]], dtype=np.float32)
    v = np.array([[[[4.0], [8.0]]]], dtype=np.float32)
    out, lse = oracle.decode(q, k, v)
    assert abs(out[0, 0, 0] - 7.0) < 5e-8
    assert abs(lse[0, 0] - math.log(4.0)) < 5e-8


# --------------------------------------------------------------------------
# P4: closed forms and bounds
# --------------------------------------------------------------------------

def test_constant_keys_give_mean_of_values():
    rng = np.random.default_rng(3)
    n, d = 1000, 8
    q = rng.standard_normal((1, 1, d)).astype(np.float32)
    krow = rng.standard_normal(d).astype(np.float32)
    k = np.broadcast_to(krow, (1, 1, n, d)).copy()
    v = rng.standard_normal((1, 1, n, d)).astype(np.float32)
    out, lse = oracle.decode(q, k, v)
    s = float(np.dot(q[0, 0].astype(np.float64), krow.astype(np.float64))) / math.sqrt(d)
    np.testing.assert_allclose(out[0, 0], v[0, 0].astype(np.float64).mean(axis=0), rtol=1e-12, atol=1e-13)
    assert abs(lse[0, 0] - (s + math.log(n))) < 1e-12 * max(1, abs(s + math.log(n)))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_one_dominant_key_selects_its_value_row(dtype):
    # q = 8 * e_0, every key row has |k_0| <= 1 except row j* with k_0 = 64, so the
    # logit gap is at least (64 - 1) * 8 / sqrt(d) = 126 >> 40: out = V[j*] to ~e^-126.
    rng = np.random.default_rng(4)
    n, d, jstar = 4096, 16, 1234
    q = np.zeros((1, 1, d), dtype=np.float32)
    q[0, 0, 0] = 8.0
    k = rng.uniform(-1, 1, (1, 1, n, d)).astype(np.float32)
    k[0, 0, jstar, 0] = 64.0
    v = rng.standard_normal((1, 1, n, d)).astype(np.float32)
    if dtype == "bf16":
        q, k, v = (W.f32_to_bf16_bits(x) for x in (q, k, v))
    out, lse = oracle.decode(q, k, v)
    np.testing.assert_allclose(out[0, 0], widen(v)[0, 0, jstar], rtol=0, atol=1e-12)
    s_star = 8.0 * 64.0 / math.sqrt(d)
    assert abs(lse[0, 0] - s_star) < 1e-12 * s_star


def test_single_token_and_empty_sequence():
    inp = W.random_decode(B=2, Hq=2, Hkv=1, N=5, d=4, dtype="f32", seed=9, seqlens=[1, 0])
    out, lse = oracle.decode(inp.q, inp.k, inp.v, inp.seqlens)
    for h in range(2):
        s0 = float(np.dot(inp.q[0, h].astype(np.float64), inp.k[0, 0, 0].astype(np.float64))) / 2.0
        np.testing.assert_allclose(out[0, h], inp.v[0, 0, 0].astype(np.float64), rtol=0, atol=0)
        assert abs(lse[0, h] - s0) < 1e-15 * max(1.0, abs(s0))
    assert np.all(out[1] == 0) and np.all(np.isneginf(lse[1]))


def test_constant_and_shifted_values():
    inp = W.random_decode(B=1, Hq=4, Hkv=2, N=300, d=8, dtype="f32", seed=12, seqlens=[300])
    # values on a 2^-10 grid, so that v + 2 below is exact in float32
    inp.v = (np.round(inp.v * 1024) / 1024).astype(np.float32)
    out, lse = oracle.decode(inp.q, inp.k, inp.v, inp.seqlens)
    # V rows all equal to c: out = c exactly up to rounding
    c = np.arange(8, dtype=np.float32) - 3.5
    vc = np.broadcast_to(c, inp.v.shape).copy()
    oc, lc = oracle.decode(inp.q, inp.k, vc, inp.seqlens)
    np.testing.assert_allclose(oc, np.broadcast_to(c.astype(np.float64), oc.shape), rtol=0, atol=1e-13)
    np.testing.assert_array_equal(lc, lse)  # lse does not depend on V
    # V + 2: out + 2 (2 is exact in float32, so the shifted values are exact)
    os_, ls_ = oracle.decode(inp.q, inp.k, (inp.v + np.float32(2.0)).astype(np.float32), inp.seqlens)
    np.testing.assert_allclose(os_, out + 2.0, rtol=0, atol=1e-13)
    np.testing.assert_array_equal(ls_, lse)


def test_token_permutation_and_bounds():
    inp = W.random_decode(B=1, Hq=2, Hkv=1, N=257, d=8, dtype="bf16", seed=13, seqlens=[257])
    out, lse = oracle.decode(inp.q, inp.k, inp.v, inp.seqlens)
    perm = np.random.default_rng(1).permutation(257)
    po, pl = oracle.decode(inp.q, inp.k[:, :, perm].copy(), inp.v[:, :, perm].copy(), inp.seqlens)
    np.testing.assert_allclose(po, out, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(pl, lse, rtol=1e-14)
    vf = widen(inp.v)[0, 0]
    kf = widen(inp.k)[0, 0]
    for h in range(2):
        s = kf @ widen(inp.q)[0, h] / math.sqrt(8)
        M = s.max()
        assert M - 1e-12 <= lse[0, h] <= M + math.log(257) + 1e-12
        assert np.all(out[0, h] >= vf.min(axis=0) - 1e-12) and np.all(out[0, h] <= vf.max(axis=0) + 1e-12)


# --------------------------------------------------------------------------
# P5: a library routine in float64
# --------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_matches_torch_sdpa_float64(dtype):
    B, Hq, Hkv, N, d = 2, 8, 2, 513, 64
    inp = W.random_decode(B=B, Hq=Hq, Hkv=Hkv, N=N, d=d, dtype=dtype, seed=21, seqlens=[513, 200])
    out, lse = oracle.decode(inp.q, inp.k, inp.v, inp.seqlens)
    qf, kf, vf = (torch.from_numpy(widen(x)) for x in (inp.q, inp.k, inp.v))
    G = Hq // Hkv
    for b in range(B):
        n = int(inp.seqlens[b])
        kk = kf[b, :, :n].repeat_interleave(G, dim=0)  # [Hq, n, d]
        vv = vf[b, :, :n].repeat_interleave(G, dim=0)
        qq = qf[b].unsqueeze(1)                          # [Hq, 1, d]
        ref = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv).squeeze(1)
        scores = torch.matmul(qq, kk.transpose(-1, -2).contiguous()).squeeze(1) / math.sqrt(d)
        ref_lse = torch.logsumexp(scores, dim=-1)
        np.testing.assert_allclose(out[b], ref.numpy(), rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(lse[b], ref_lse.numpy(), rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------
# P3: any chunking and any binary tree give the unchunked result
# --------------------------------------------------------------------------

@pytest.mark.parametrize("n", [1, 2, 3, 5, 6])
def test_every_chunking_and_tree_shape_matches_unchunked(n):
    inp = W.random_decode(B=1, Hq=2, Hkv=1, N=n, d=3, dtype="f32", seed=100 + n, seqlens=[n])
    out, lse = oracle.decode(inp.q, inp.k, inp.v, inp.seqlens)
    for bounds in compositions(n):
        parts = [window_state(inp.q, inp.k, inp.v, inp.seqlens, a, b) for (a, b) in bounds]
        for h in range(2):
            leaves = [oracle.from_normalized(po[0, h], pl[0, h]) for (po, pl) in parts]
            n_trees = 0
            for root in all_trees(leaves):
                o, l = oracle.finalize(root)
                np.testing.assert_allclose(o, out[0, h], rtol=1e-13, atol=1e-14)
                assert abs(l - lse[0, h]) <= 1e-13 * max(1.0, abs(lse[0, h]))
                n_trees += 1
            assert n_trees == math.comb(2 * (len(leaves) - 1), len(leaves) - 1) // len(leaves)
            # the definition-form combine gives the same state
            co, cl = oracle.combine(np.stack([p[0][0, h] for p in parts]).astype(np.float32),
                                    np.array([p[1][0, h] for p in parts], dtype=np.float32))
            # partials were rounded to float32 for combine: compare at float32 accuracy
            np.testing.assert_allclose(co, out[0, h], rtol=1e-6, atol=1e-6)
            assert abs(cl - lse[0, h]) <= 1e-6 * max(1.0, abs(lse[0, h]))


def test_page_form_states_merge_to_unchunked():
    # build (o, l, m) states from raw token windows (the page's local partial state),
    # fold them in random orders and random tree arities, normalise at the root
    n, d = 40, 8
    inp = W.random_decode(B=1, Hq=1, Hkv=1, N=n, d=d, dtype="f32", seed=7, seqlens=[n])
    out, lse = oracle.decode(inp.q, inp.k, inp.v, inp.seqlens)
    qf, kf, vf = widen(inp.q)[0, 0], widen(inp.k)[0, 0], widen(inp.v)[0, 0]
    s = kf @ qf / math.sqrt(d)
    rng = np.random.default_rng(0)
    for trial in range(20):
        cuts = np.sort(rng.choice(np.arange(1, n), size=rng.integers(1, 12), replace=False))
        bounds = list(zip(np.r_[0, cuts], np.r_[cuts, n]))
        states = []
        for a, b in bounds:
            m = s[a:b].max()
            p = np.exp(s[a:b] - m)
            states.append((p @ vf[a:b], p.sum(), m))
        order = rng.permutation(len(states))
        root, levels = oracle.tree_fold([states[i] for i in order], arity=int(rng.integers(2, 5)))
        o, l = oracle.finalize(root)
        np.testing.assert_allclose(o, out[0, 0], rtol=1e-13, atol=1e-14)
        assert abs(l - lse[0, 0]) <= 1e-13 * abs(lse[0, 0])
        chain, steps = oracle.chain_fold(states)
        o2, l2 = oracle.finalize(chain)
        np.testing.assert_allclose(o2, out[0, 0], rtol=1e-13, atol=1e-14)
        assert steps == len(states) - 1


def test_merge_of_empty_states_is_identity():
    d = 4
    e = oracle.empty_state(d)
    a = (np.arange(d, dtype=np.float64), 2.5, 1.25)
    for x, y in [(e, a), (a, e)]:
        o, l, m = oracle.merge(x, y)
        np.testing.assert_array_equal(o, a[0])
        assert l == a[1] and m == a[2]
    o, l, m = oracle.merge(e, e)
    assert np.all(o == 0) and l == 0 and m == -np.inf
    o, l = oracle.finalize(oracle.merge(e, e))
    assert np.all(o == 0) and l == -np.inf


def test_tree_depths_printed_on_the_page():
    with open(os.path.join(HERE, "golden", "tree_depths.json")) as f:
        g = json.load(f)
    for case in g["cases"]:
        leaves = [oracle.from_normalized(np.zeros(2), 0.0)] * case["P"]
        _, levels = oracle.tree_fold(leaves, arity=case["arity"])
        _, hops = oracle.chain_fold(leaves)
        assert levels == case["tree_levels"]
        assert hops == case["ring_hops"]


# --------------------------------------------------------------------------
# combine: closed forms and edge cases of the definition form
# --------------------------------------------------------------------------

def test_combine_closed_forms():
    rng = np.random.default_rng(8)
    d = 16
    po = rng.standard_normal((3, 5, d)).astype(np.float32)
    # equal lse: the mean of the states, lse + ln 5
    pl = np.full((3, 5), 2.0, dtype=np.float32)
    o, l = oracle.combine(po, pl)
    np.testing.assert_allclose(o, po.astype(np.float64).mean(axis=1), rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(l, 2.0 + math.log(5), rtol=1e-14)
    # one state 60 above the rest: that state's o
    pl = rng.uniform(-3, 3, (3, 5)).astype(np.float32)
    pl[:, 2] = 70.0
    o, l = oracle.combine(po, pl)
    np.testing.assert_allclose(o, po[:, 2].astype(np.float64), rtol=0, atol=1e-20 + 1e-25)
    np.testing.assert_allclose(l, 70.0, rtol=1e-15)
    # n_parts = 1: identity
    o, l = oracle.combine(po[:, :1], pl[:, :1])
    np.testing.assert_array_equal(o, po[:, 0].astype(np.float64))
    np.testing.assert_array_equal(l, pl[:, 0].astype(np.float64))


def test_combine_empty_states():
    d = 8
    po = np.ones((2, 4, d), dtype=np.float32)
    pl = np.full((2, 4), -np.inf, dtype=np.float32)
    pl[0, 1] = 3.0
    po[0, 1] = 5.0
    o, l = oracle.combine(po, pl)
    np.testing.assert_array_equal(o[0], np.full(d, 5.0))
    assert l[0] == 3.0
    assert np.all(o[1] == 0) and l[1] == -np.inf


def test_combine_of_decode_windows_equals_decode():
    inp = W.random_decode(B=2, Hq=4, Hkv=2, N=1000, d=32, dtype="bf16", seed=31, seqlens=[1000, 333])
    out, lse = oracle.decode(inp.q, inp.k, inp.v, inp.seqlens)
    chunk = 128
    P = 8
    po = np.zeros((2, 4, P, 32), dtype=np.float32)
    pl = np.zeros((2, 4, P), dtype=np.float32)
    for i in range(P):
        o, l = window_state(inp.q, inp.k, inp.v, inp.seqlens, i * chunk, (i + 1) * chunk)
        po[:, :, i] = o
        pl[:, :, i] = l
    assert np.isneginf(pl[1, :, 3:]).all()  # chunks past the end of sequence 1 are empty
    co, cl = oracle.combine(po, pl)
    np.testing.assert_allclose(co, out, rtol=0, atol=1e-6)
    np.testing.assert_allclose(cl, lse, rtol=1e-7)


# --------------------------------------------------------------------------
# the pins catch plausible slips: mutate the oracle source, rebuild, re-run
# --------------------------------------------------------------------------

MUTATIONS = [
    ("dropped scale", "s[j - t0] = acc * scale;", "s[j - t0] = acc;"),
    ("GQA index h % Hkv", "g = h / group;", "g = h % Hkv;"),
    ("K transposed", "load_elem(k, dtype, kvoff + j * d + c)", "load_elem(k, dtype, kvoff + c * N + j)"),
    ("lse sign", "lse[r] = M + log(Z);", "lse[r] = M - log(Z);"),
    ("max not subtracted in weights", "const double w = exp(s[j - t0] - M);", "const double w = exp(s[j - t0]);"),
    ("no normalisation", "for (int64_t c = 0; c < d; ++c) o[c] /= Z;", ""),
    ("V row off by one", "o[c] += w * load_elem(v, dtype, kvoff + j * d + c);",
     "o[c] += w * load_elem(v, dtype, kvoff + (j + 1 < t1 ? j + 1 : j) * d + c);"),
]


def _build_mutant(tmp_path, old, new):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "oracle.c")).read()
    assert src.count(old) == 1, old
    path = tmp_path / "mut.c"
    path.write_text(src.replace(old, new))
    lib = tmp_path / "libmut.so"
    subprocess.run(["gcc", "-O1", "-fPIC", "-shared", "-std=c11", str(path), "-o", str(lib), "-lm"], check=True)
    return ctypes.CDLL(str(lib))


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistakes_are_caught(tmp_path, name, old, new):
    lib = _build_mutant(tmp_path, old, new)
    p, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.oracle_decode.argtypes = [p, p, p, i32, i64, i64, i64, i64, i64, p, i64, i64, p, i64, p, p]
    inp = W.random_decode(B=2, Hq=4, Hkv=2, N=7, d=3, dtype="f32", seed=1, seqlens=[7, 4])
    out = np.zeros((8, 3))
    lse = np.zeros(8)
    sl = inp.seqlens.astype(np.int32)
    rc = lib.oracle_decode(inp.q.ctypes.data, inp.k.ctypes.data, inp.v.ctypes.data, 0, 2, 4, 2, 7, 3,
                           sl.ctypes.data, 0, -1, None, 8, out.ctypes.data, lse.ctypes.data)
    assert rc == 0
    bo, bl = brute_force(inp.q, inp.k, inp.v, inp.seqlens)
    agree = np.allclose(out.reshape(2, 4, 3), bo, rtol=1e-12, atol=1e-13) and \
        np.allclose(lse.reshape(2, 4), bl, rtol=1e-12, atol=1e-13)
    assert not agree, f"planted mistake '{name}' went unnoticed by the brute-force pin"
