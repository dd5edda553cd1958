"""GPU parity: the HIP path through the C ABI against the float64 oracle.

Every case is compared element by element over every output, the
workload-sized ones (128k to 1M tokens, ragged batches, the full merge
workload) included, in the launch configuration the benchmark times. Tolerances are in gpu_helpers.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import softmax_tree_reduction_amd as ta
import workloads as W
from gpu_helpers import assert_close, dev_tensor, log, upload

pytestmark = pytest.mark.gpu


def run_decode(inp, chunk, layout="bhnd"):
    q, k, v, sl = upload(inp)
    if layout == "bnhd":  # token-major cache [B, N, Hkv, d] seen through a permuted view
        k = k.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
        v = v.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    out, lse = ta.decode(q, k, v, sl, chunk=chunk)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def check_small(inp, chunk, layout="bhnd", what=""):
    log(f"case {what}: B={inp.q.shape[0]} Hq={inp.q.shape[1]} Hkv={inp.k.shape[1]} N={inp.k.shape[2]} "
        f"d={inp.q.shape[2]} seqlens={list(inp.seqlens)} chunk={chunk} layout={layout}")
    out, lse = run_decode(inp, chunk, layout)
    ref_o, ref_l = oracle.decode(inp.q, inp.k, inp.v, inp.seqlens)
    dtype = "bf16" if inp.q.dtype == np.uint16 else "f32"
    return assert_close(out, lse, ref_o, ref_l, dtype, what)


# ---------------------------------------------------------------- small, exhaustive

def test_tiny_f32_workload_full():
    wl = W.WORKLOADS["tiny_f32"]
    inp = W.make_decode_inputs(wl, 1)
    err, lerr = check_small(inp, wl.chunk, what="tiny_f32")
    log(f"tiny_f32: max abs out err {err:.2e}, max rel lse err {lerr:.2e}")


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("f32", 64), ("f32", 128)])
@pytest.mark.parametrize("chunk", [1, 37, 256, 375, 2048, 100000])
def test_ragged_tails_all_dtypes(dtype, d, chunk):
    # 3000 tokens: several tiles, a ragged tail, one empty sequence, one shorter than a block
    N = 3000
    inp = W.random_decode(B=4, Hq=8, Hkv=2, N=N, d=d, dtype=dtype, seed=3, seqlens=[3000, 1777, 0, 5])
    check_small(inp, chunk, what=f"ragged {dtype} d={d} chunk={chunk}")


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("f32", 128)])
@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (8, 4), (16, 4), (32, 4), (12, 4), (24, 4), (5, 1)])
def test_gqa_group_sizes(Hq, Hkv, dtype, d):
    # G = 1, 2, 4, 8 run one workgroup per group; G = 3 and 6 split the group; G = 5 (MQA-like).
    # bf16 d = 64 has 8-lane rows, f32 d = 128 32-lane rows: each row width meets each head count.
    inp = W.random_decode(B=2, Hq=Hq, Hkv=Hkv, N=1500, d=d, dtype=dtype, seed=Hq * 10 + Hkv,
                          seqlens=[1500, 999])
    check_small(inp, 512, what=f"GQA {Hq}/{Hkv} {dtype} d={d}")


def test_token_major_strided_cache():
    inp = W.random_decode(B=2, Hq=8, Hkv=2, N=2000, d=128, dtype="bf16", seed=8, seqlens=[2000, 1234])
    check_small(inp, 300, layout="bnhd", what="token-major cache")


@pytest.mark.parametrize("dtype,d", [("bf16", 64), ("bf16", 128), ("f32", 128)])
def test_token_stride_at_the_limit(dtype, d):
    # Rows 256 MiB - 256 B apart, just under the largest token stride the library takes:
    # one wave-wide load then spans up to 7 such strides (bf16 d = 64), the largest
    # offsets the partial kernel forms. Two full blocks and a partial one, in one chunk
    # and in chunks of one block; the bytes between rows are never written.
    bt = BLOCK_TOKENS[(dtype, d)]
    N = 2 * bt + 3
    inp = W.random_decode(B=1, Hq=4, Hkv=1, N=N, d=d, dtype=dtype, seed=d + N, seqlens=[N])
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    es = 2 if dtype == "bf16" else 4
    stride = ((1 << 28) - 256) // es  # elements
    q, kc, vc, _ = upload(inp)
    log(f"token stride limit: {dtype} d={d} N={N} stride={stride * es} B, {N * stride * es / 2**30:.1f} GiB per tensor")
    k_big = torch.empty(N * stride, dtype=tdt, device="cuda")
    v_big = torch.empty(N * stride, dtype=tdt, device="cuda")
    k_big.view(N, stride)[:, :d] = kc[0, 0]
    v_big.view(N, stride)[:, :d] = vc[0, 0]
    k = k_big.as_strided((1, 1, N, d), (N * stride, N * stride, stride, 1))
    v = v_big.as_strided((1, 1, N, d), (N * stride, N * stride, stride, 1))
    ref_o, ref_l = oracle.decode(inp.q, inp.k, inp.v, inp.seqlens)
    for chunk in (N, bt):
        out, lse = ta.decode(q, k, v, None, chunk=chunk)
        torch.cuda.synchronize()
        assert_close(out.cpu().numpy(), lse.cpu().numpy(), ref_o, ref_l, dtype, what=f"stride limit chunk {chunk}")
    del k, v, k_big, v_big
    torch.cuda.empty_cache()


def test_peaked_keys_small():
    wl = W.DecodeWorkload("peaked-small", B=2, Hq=32, Hkv=8, d=128, N=8192, chunk=1024, dtype="bf16",
                          spike_frac=0.01, spike_scale=8.0)
    inp = W.make_decode_inputs(wl, 4)
    check_small(inp, wl.chunk, what="peaked small")


def test_single_chunk_pins_partial_kernel():
    # chunk >= n: one partial state per row, the merge is the identity
    inp = W.random_decode(B=2, Hq=8, Hkv=2, N=4000, d=128, dtype="bf16", seed=9, seqlens=[4000, 2500])
    check_small(inp, 4096, what="single chunk")


def test_partial_states_match_oracle_windows():
    # 8 chunks per row of a ragged batch: the chunk order is rotated per row across
    # the XCDs, and every state must still land in its own slot
    inp = W.random_decode(B=3, Hq=8, Hkv=2, N=2400, d=128, dtype="bf16", seed=10, seqlens=[2400, 700, 2399])
    chunk = 300
    q, k, v, sl = upload(inp)
    po, pl = ta.partial(q, k, v, sl, chunk=chunk)
    torch.cuda.synchronize()
    po, pl = po.cpu().numpy(), pl.cpu().numpy()
    P = -(-2400 // chunk)
    assert po.shape == (3, 8, P, 128) and P == 8
    for i in range(P):
        ro, rl = oracle.decode(inp.q, inp.k, inp.v, inp.seqlens, t_begin=i * chunk, t_end=(i + 1) * chunk)
        assert_close(po[:, :, i], pl[:, :, i], ro, rl, "bf16", what=f"partial {i}")
    # merging them with ta_combine reproduces ta_decode bit for bit
    out, lse = ta.combine(torch.from_numpy(po).cuda(), torch.from_numpy(pl).cuda())
    out2, lse2 = ta.decode(q, k, v, sl, chunk=chunk)
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(lse, lse2)


@pytest.mark.parametrize("B,P,Hq,Hkv,d,chunk", [
    (5, 8, 32, 8, 128, 64), (5, 32, 32, 8, 128, 64), (5, 33, 32, 8, 128, 64), (5, 64, 32, 8, 128, 64),
    (64, 33, 32, 8, 128, 64), (72, 32, 32, 8, 128, 64), (72, 64, 32, 8, 128, 64), (200, 33, 32, 8, 128, 32),
    (520, 32, 8, 8, 64, 16), (520, 33, 8, 8, 64, 16), (520, 40, 8, 8, 64, 16)])
def test_ragged_chunk_orders_match_oracle_windows(B, P, Hq, Hkv, d, chunk):
    # Ragged grids of at most 64 sequences take the compacted order (the workgroups
    # with work first; those after them write the empty states of sequences without
    # tokens). Larger ones with 8 head groups per sequence and at most 32 chunks per
    # row are walked chunk-major, the others with the chunk index fastest (rotated per
    # row when the row has a multiple of 8 chunks). Every state must land in its own
    # slot. At B = 5,
    # P = 64 the grid (2560 workgroups) has more than 8 per CU of a 256-CU device, so
    # the launch also reserves LDS to keep two workgroups per CU.
    N = P * chunk
    base = [N, min(700, N - 3), N - 1, 0, 65]
    lens = [base[b % 5] if b % 3 else (b * 7919) % (N + 1) for b in range(B)]
    inp = W.random_decode(B=B, Hq=Hq, Hkv=Hkv, N=N, d=d, dtype="bf16", seed=P + B, seqlens=lens)
    log(f"chunk orders: B={B} P={P} N={N} lens={lens[:8]}...")
    q, k, v, sl = upload(inp)
    po, pl = ta.partial(q, k, v, sl, chunk=chunk)
    out, lse = ta.decode(q, k, v, sl, chunk=chunk)
    torch.cuda.synchronize()
    po, pl = po.cpu().numpy(), pl.cpu().numpy()
    for i in range(P):
        ro, rl = oracle.decode(inp.q, inp.k, inp.v, inp.seqlens, t_begin=i * chunk, t_end=(i + 1) * chunk)
        assert_close(po[:, :, i], pl[:, :, i], ro, rl, "bf16", what=f"B={B} P={P} state {i}")
    ref_o, ref_l = oracle.decode(inp.q, inp.k, inp.v, inp.seqlens)
    assert_close(out.cpu().numpy(), lse.cpu().numpy(), ref_o, ref_l, "bf16", what=f"B={B} P={P} decode")


# tokens in one wave-wide block: 4 tokens per lane x the rows a wave-wide load covers
# (64 lanes / the 16-byte segments of a row)
BLOCK_TOKENS = {("bf16", 128): 16, ("bf16", 64): 32, ("f32", 128): 8, ("f32", 64): 16}


@pytest.mark.parametrize("grid", ["one per CU", "small"])
@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("f32", 128), ("f32", 64)])
def test_partial_states_across_block_loop_phases(dtype, d, grid):
    # Each wave streams its blocks in turns of the register ring: turns whose prefetches
    # all lie inside the chunk issue them unconditionally, the one or two blocks left
    # after them run as straight-line code per case, and one wave then takes the
    # chunk's partial block. Chunks of 0 to 25 full
    # blocks, with and without a partial block, put every wave in every phase, with
    # 4 waves per workgroup (a grid of one workgroup per CU) and with 8 (a small grid).
    # Every state is checked against the oracle over its own window.
    bt = BLOCK_TOKENS[(dtype, d)]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    B, Hq, Hkv = (cus // 64, 32, 8) if grid == "one per CU" else (1, 8, 2)
    if grid == "one per CU" and cus % 64:
        pytest.skip(f"{cus} CUs is no multiple of 64")
    for nfull in (0, 1, 3, 8, 9, 11, 12, 16, 17, 25):
        for tail in (0, 3):
            chunk = nfull * bt + tail
            if chunk == 0:
                continue
            N = 8 * chunk  # 8 chunks per row: 8 x 8 head groups x B workgroups
            lens = [N, N - chunk // 2 - 1, 3 * chunk + 1, N][:B] if B > 1 else [N - 1]
            lens += [N] * (B - len(lens))
            inp = W.random_decode(B=B, Hq=Hq, Hkv=Hkv, N=N, d=d, dtype=dtype, seed=nfull * 10 + tail, seqlens=lens)
            log(f"loop phases: {dtype} d={d} {grid} chunk={chunk} ({nfull} blocks + {tail}) B={B} lens={lens}")
            q, k, v, sl = upload(inp)
            po, pl = ta.partial(q, k, v, sl, chunk=chunk)
            torch.cuda.synchronize()
            po, pl = po.cpu().numpy(), pl.cpu().numpy()
            for i in range(8):
                ro, rl = oracle.decode(inp.q, inp.k, inp.v, inp.seqlens, t_begin=i * chunk, t_end=(i + 1) * chunk)
                assert_close(po[:, :, i], pl[:, :, i], ro, rl, dtype, what=f"chunk {chunk} state {i}")


@pytest.mark.parametrize("B,Hq,Hkv,N,d,chunk,seqlens", [
    # 48 workgroups: write-back state stores
    (3, 8, 2, 2400, 128, 300, [2400, 700, 0]),
    # 8192 and 16384 workgroups (more than 8 per compute unit): nontemporal state stores
    (4, 32, 8, 4096, 128, 16, [4096, 9, 0, 17]),
    (8, 8, 8, 2048, 64, 8, [2048, 1, 0, 9, 1000, 8, 2047, 17]),
])
def test_partial_writes_every_slot(B, Hq, Hkv, N, d, chunk, seqlens):
    # Chunks past a sequence's end hold the empty state (0, -inf), written by the
    # row's non-empty chunks (a row with one or two of them writes hundreds), or by
    # the chunk itself when the row has no tokens. The buffers start as NaN, so a
    # slot nobody wrote fails.
    inp = W.random_decode(B=B, Hq=Hq, Hkv=Hkv, N=N, d=d, dtype="bf16", seed=B * 100 + chunk, seqlens=seqlens)
    P = -(-N // chunk)
    log(f"partial slots: B={B} Hq={Hq} Hkv={Hkv} N={N} d={d} chunk={chunk} P={P} workgroups={P * B * Hq // min(Hq // Hkv, 8)}")
    q, k, v, sl = upload(inp)
    po = torch.full((B, Hq, P, d), float("nan"), dtype=torch.float32, device="cuda")
    pl = torch.full((B, Hq, P), float("nan"), dtype=torch.float32, device="cuda")
    ta.partial(q, k, v, sl, chunk=chunk, partial_o=po, partial_lse=pl)
    torch.cuda.synchronize()
    po, pl = po.cpu().numpy(), pl.cpu().numpy()
    for b, n in enumerate(seqlens):
        nb = -(-n // chunk)
        assert np.all(po[b, :, nb:] == 0.0) and np.all(np.isneginf(pl[b, :, nb:])), f"row {b}: empty slots"
        assert np.all(np.isfinite(po[b, :, :nb])) and np.all(np.isfinite(pl[b, :, :nb])), f"row {b}: unwritten slot"
    for i in range(max(-(-n // chunk) for n in seqlens)):
        ro, rl = oracle.decode(inp.q, inp.k, inp.v, inp.seqlens, t_begin=i * chunk, t_end=(i + 1) * chunk)
        assert_close(po[:, :, i], pl[:, :, i], ro, rl, "bf16", what=f"partial {i}")


@pytest.mark.parametrize("chunk", [64, 16])
def test_partial_clamps_out_of_range_seqlens(chunk):
    # lengths below 0 or above N act as 0 and N: every slot, the empty ones included,
    # holds what the clamped lengths give (chunk 16: 8192 workgroups, nontemporal stores)
    N = 4096 if chunk == 16 else 1000
    inp = W.random_decode(B=4, Hq=32, Hkv=8, N=N, d=128, dtype="bf16", seed=chunk, seqlens=[N, 0, 3, N])
    q, k, v, _ = upload(inp)
    P = -(-N // chunk)
    res = []
    for lens in ([N + 1000, -5, 3, 2**31 - 1], [N, 0, 3, N]):
        po = torch.full((4, 32, P, 128), float("nan"), dtype=torch.float32, device="cuda")
        pl = torch.full((4, 32, P), float("nan"), dtype=torch.float32, device="cuda")
        ta.partial(q, k, v, torch.tensor(lens, dtype=torch.int32, device="cuda"), chunk=chunk,
                   partial_o=po, partial_lse=pl)
        res.append((po, pl))
    torch.cuda.synchronize()
    assert not torch.isnan(res[1][0]).any() and not torch.isnan(res[1][1]).any()
    assert torch.equal(res[0][0], res[1][0]) and torch.equal(res[0][1], res[1][1])


@pytest.mark.parametrize("B,seqlens", [
    (2, [1000, 0]),                                   # 1024 workgroups: write-back state stores
    (4, [4096, 1, 0, 1000]),                          # 2048 workgroups: write-back state stores
    (8, [4096, 1, 0, 1000, 64, 65, 4095, 2000]),      # 4096 workgroups: nontemporal state stores
])
def test_decode_never_reads_chunks_past_the_end(B, seqlens):
    # With seqlens, ta_decode leaves the states of chunks past a sequence's end
    # unwritten: the merge must not read them. A first call on the same stream and
    # shapes, at full length, fills every slot of the workspace with a state whose
    # lse (about 30, from keys scaled by 8) dwarfs any real one here (1 to 9) and
    # whose o is 1024: one stale slot read would pull that row's output to 1024.
    Hq, Hkv, N, d, chunk = 32, 8, 4096, 128, 64
    log(f"stale workspace: B={B} N={N} chunk={chunk} seqlens={seqlens}")
    inp = W.random_decode(B=B, Hq=Hq, Hkv=Hkv, N=N, d=d, dtype="bf16", seed=B + 7, seqlens=seqlens)
    q, k, v, sl = upload(inp)
    gen = torch.Generator(device="cuda").manual_seed(B)
    big_k = (torch.randn(k.shape, generator=gen, device="cuda") * 8).to(torch.bfloat16)
    big_v = torch.full_like(v, 1024.0)
    full = torch.full((B,), N, dtype=torch.int32, device="cuda")
    out, lse = ta.decode(q, big_k, big_v, full, chunk=chunk)
    torch.cuda.synchronize()
    assert torch.allclose(out, torch.full_like(out, 1024.0)) and (lse > 20).all(), "poisoning call"
    out, lse = ta.decode(q, k, v, sl, chunk=chunk)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.decode(inp.q, inp.k, inp.v, inp.seqlens)
    assert_close(out.cpu().numpy(), lse.cpu().numpy(), ref_o, ref_l, "bf16", what="after a poisoned workspace")


@pytest.mark.parametrize("n_parts", [1, 3, 5, 7, 64, 128, 200, 1000, 20000])
@pytest.mark.parametrize("d", [128, 64])
def test_combine_against_oracle(n_parts, d):
    # 20000 leaves take three passes (128 or 256 leaves per workgroup)
    wl = W.CombineWorkload("c", B=3, H=5 if n_parts < 10000 else 1, n_parts=n_parts, d=d)
    ci = W.make_combine_inputs(wl, n_parts + d)
    pl = ci.partial_lse.copy()
    rng = np.random.default_rng(n_parts)
    pl[rng.random(pl.shape) < 0.2] = -np.inf   # empty states mixed in
    pl[1, -1] = -np.inf                        # a row with no state at all
    pl[0, 0] = rng.uniform(-80, 80, n_parts).astype(np.float32)  # a wide spread
    log(f"combine n_parts={n_parts} d={d}")
    out, lse = ta.combine(dev_tensor(ci.partial_o), dev_tensor(pl))
    torch.cuda.synchronize()
    ro, rl = oracle.combine(ci.partial_o, pl)
    assert_close(out.cpu().numpy(), lse.cpu().numpy(), ro, rl, "f32", what=f"combine {n_parts}")


def combine_inputs_with_empties(B, H, n_parts, d, seed):
    ci = W.make_combine_inputs(W.CombineWorkload("c", B=B, H=H, n_parts=n_parts, d=d), seed)
    pl = ci.partial_lse.copy()
    rng = np.random.default_rng(seed)
    pl[rng.random(pl.shape) < 0.2] = -np.inf   # empty states mixed in
    pl[B - 1, H - 1] = -np.inf                 # a row with no state at all
    pl[0, 0] = rng.uniform(-80, 80, n_parts).astype(np.float32)  # a wide spread
    return ci.partial_o, pl


def arity_span(d, arity):
    """Leaves one launch of ta_combine_k takes (either head dimension): the largest
    power K^j of the arity with K^(j-1) <= 64 first-level nodes."""
    span = arity
    while span <= 64:
        span *= arity
    return span


@pytest.mark.parametrize("arity", [2, 3, 4, 5, 7, 8, 16])
@pytest.mark.parametrize("n_parts", [1, 7, 16, 17, 64, 65, 300, 5000])
@pytest.mark.parametrize("d", [128, 64])
def test_combine_k_against_oracle(arity, n_parts, d):
    po, pl = combine_inputs_with_empties(3, 4, n_parts, d, 7 * n_parts + arity)
    log(f"combine_k arity={arity} n_parts={n_parts} d={d}")
    out, lse = ta.combine(dev_tensor(po), dev_tensor(pl), arity=arity)
    torch.cuda.synchronize()
    ro, rl = oracle.combine(po, pl)
    assert_close(out.cpu().numpy(), lse.cpu().numpy(), ro, rl, "f32", what=f"combine_k {arity} {n_parts}")


@pytest.mark.parametrize("d", [128, 64])
def test_combine_k_arity_two_is_the_binary_tree(d):
    # within one launch both kernels run the same binary tree with the same
    # operand order, so the results agree bit for bit; at d = 128 both take 128
    # leaves per launch, so longer rows split into the same passes too
    more = (1000, 20000) if d == 128 else ()
    for n_parts in (1, 2, 3, 13, 32, arity_span(d, 2)) + more:
        po, pl = combine_inputs_with_empties(2, 6, n_parts, d, 100 + n_parts)
        log(f"combine_k arity=2 vs binary n_parts={n_parts} d={d}")
        a = ta.combine(dev_tensor(po), dev_tensor(pl), arity=2)
        b = ta.combine(dev_tensor(po), dev_tensor(pl))
        torch.cuda.synchronize()
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1]), n_parts


@pytest.mark.parametrize("arity", [2, 3, 4, 16])
@pytest.mark.parametrize("d", [128, 64])
def test_combine_k_passes_are_subtrees(arity, d):
    # A row longer than one launch takes is merged per aligned group of `span`
    # leaves (a power of the arity, so each group is a whole subtree), and the
    # group roots are merged by the same tree: the same as doing it by hand.
    span = arity_span(d, arity)
    n_parts = span * span + 3 * span + 5     # three passes: span + 4 roots, then 2
    po, pl = combine_inputs_with_empties(1, 2, n_parts, d, 300 + arity)
    log(f"combine_k passes arity={arity} d={d} span={span} n_parts={n_parts}")
    po_d, pl_d = dev_tensor(po), dev_tensor(pl)
    direct = ta.combine(po_d, pl_d, arity=arity)
    level = (po_d, pl_d)
    while level[0].shape[2] > span:
        n = level[0].shape[2]
        roots = [ta.combine(level[0][:, :, g:g + span].contiguous(), level[1][:, :, g:g + span].contiguous(),
                            arity=arity) for g in range(0, n, span)]
        level = (torch.stack([r[0] for r in roots], 2), torch.stack([r[1] for r in roots], 2))
    by_hand = ta.combine(level[0], level[1], arity=arity)
    torch.cuda.synchronize()
    assert torch.equal(direct[0], by_hand[0]) and torch.equal(direct[1], by_hand[1])


@pytest.mark.parametrize("n_parts", [0, 1, 2, 7, 9, 64, 1000])
@pytest.mark.parametrize("d", [128, 64])
def test_combine_chain_against_oracle(n_parts, d):
    # 20 heads: 8 (d = 128) or 16 (d = 64) rows per workgroup, the last one ragged
    po, pl = combine_inputs_with_empties(3, 20, max(n_parts, 1), d, 11 * n_parts + d)
    log(f"combine_chain n_parts={n_parts} d={d}")
    out, lse = ta.combine(dev_tensor(po), dev_tensor(pl), n_parts=n_parts, arity="chain")
    torch.cuda.synchronize()
    ro, rl = oracle.combine(po[:, :, :n_parts], pl[:, :, :n_parts])
    assert_close(out.cpu().numpy(), lse.cpu().numpy(), ro, rl, "f32", what=f"combine_chain {n_parts}")


def test_combine_chain_long_row_within_summation_bound():
    # The chain's last leaf passes through one merge, its first through P - 1, so
    # its rounding grows like recursive summation: |error| <= (P - 1) u sum|x| for
    # each of o and l (u = 2^-24), about 2 (P - 1) u max|o_i| on o / l, where the
    # tree's bound has log2 P in place of P - 1. Checked at that bound with u
    # doubled for the exponentials; the exact case below is the sharp pin.
    n_parts, d = 20000, 128
    po, pl = combine_inputs_with_empties(2, 3, n_parts, d, 4242)
    out, lse = ta.combine(dev_tensor(po), dev_tensor(pl), arity="chain")
    torch.cuda.synchronize()
    ro, rl = oracle.combine(po, pl)
    out, lse = out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)
    full = ~np.isneginf(rl)
    bound = 4 * (n_parts - 1) * 2.0 ** -24 * np.abs(po).max()
    err = np.abs(out[full] - ro[full]).max()
    log(f"combine_chain 20000 leaves: max |out - oracle| = {err:.3e}, bound {bound:.3e}")
    assert err <= bound
    assert np.isneginf(lse[~full]).all() and (out[~full] == 0).all()
    assert (np.abs(lse[full] - rl[full]) / np.abs(rl[full])).max() <= 1e-4


@pytest.mark.parametrize("arity,n_parts", [("chain", 20000), ("chain", 5), (None, 128), (None, 77), (4, 64), (8, 64),
                                           (16, 200), (3, 81)])
def test_merge_is_exact_where_the_arithmetic_is(arity, n_parts):
    # Equal lse_i make every rescale factor exp2(0) = 1, and o_i on a 2^-6 grid
    # with |o_i| <= 2 keep every partial sum below 2^16 on that grid: each merge
    # inside one launch is exact, in any order. The root o / l is then the exact
    # mean up to the rounding of the final division, for every merge order.
    d = 128
    rng = np.random.default_rng(n_parts)
    po = (rng.integers(-128, 129, size=(2, 3, n_parts, d)) / 64.0).astype(np.float32)
    pl = np.full((2, 3, n_parts), 3.25, dtype=np.float32)
    log(f"exact merge arity={arity} n_parts={n_parts}")
    out, lse = ta.combine(dev_tensor(po), dev_tensor(pl), arity=arity)
    torch.cuda.synchronize()
    mean = po.astype(np.float64).mean(axis=2)
    err = np.abs(out.cpu().numpy() - mean)
    assert (err <= 4 * 2.0 ** -24 * np.abs(mean) + 1e-12).all(), err.max()
    assert np.allclose(lse.cpu().numpy(), 3.25 + np.log(n_parts), rtol=1e-6, atol=0)


@pytest.mark.parametrize("d", [128, 64])
def test_combine_chain_is_one_group_of_the_k_ary_tree(d):
    # up to K leaves, the arity-K tree is a single group merged left to right:
    # the chain, bit for bit
    for arity, n_parts in ((16, 1), (16, 5), (16, 16), (8, 8), (3, 3), (2, 2)):
        po, pl = combine_inputs_with_empties(2, 9, n_parts, d, 500 + n_parts)
        log(f"combine_chain vs arity {arity}, n_parts={n_parts} d={d}")
        a = ta.combine(dev_tensor(po), dev_tensor(pl), arity="chain")
        b = ta.combine(dev_tensor(po), dev_tensor(pl), arity=arity)
        torch.cuda.synchronize()
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1]), (arity, n_parts)


def test_stream_read_probe():
    # zeros XOR to zero, so the probe leaves its sink alone; odd sizes and a
    # buffer smaller than one workgroup's share run too
    sink = torch.full((1,), 7, dtype=torch.int32, device="cuda")
    for n in (16, 4096 + 16, 3 * 2**20 + 48):
        buf = torch.zeros(n, dtype=torch.uint8, device="cuda")
        ta.stream_read(buf, sink)
    torch.cuda.synchronize()
    assert sink.item() == 7


def test_combine_uses_leading_parts_only():
    ci = W.make_combine_inputs(W.CombineWorkload("c", B=2, H=3, n_parts=40, d=128), 2)
    po, pl = dev_tensor(ci.partial_o), dev_tensor(ci.partial_lse)
    out, lse = ta.combine(po, pl, n_parts=17)
    torch.cuda.synchronize()
    ro, rl = oracle.combine(ci.partial_o[:, :, :17], ci.partial_lse[:, :, :17])
    assert_close(out.cpu().numpy(), lse.cpu().numpy(), ro, rl, "f32", what="combine n_parts=17 of 40")
    out0, lse0 = ta.combine(po, pl, n_parts=0)
    torch.cuda.synchronize()
    assert torch.all(out0 == 0) and torch.all(torch.isneginf(lse0))


def test_bitwise_deterministic():
    inp = W.random_decode(B=2, Hq=32, Hkv=8, N=20000, d=128, dtype="bf16", seed=12, seqlens=[20000, 13001])
    q, k, v, sl = upload(inp)
    a = ta.decode(q, k, v, sl, chunk=1024)
    b = ta.decode(q, k, v, sl, chunk=1024)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_concurrent_threads_and_streams():
    # Serving code may call ta_decode from several host threads, each on a stream of
    # its own. Every (device, stream) pair has its own workspace, grown when a call
    # needs more; each thread cycles through shapes of different sizes, and every
    # result must be the one a single stream gives, bit for bit.
    import threading
    cases = []
    for i, (N, chunk, sl) in enumerate([(20000, 1024, [20000, 13001]), (9000, 256, [9000, 1]),
                                        (30000, 2048, [29999, 30000])]):
        inp = W.random_decode(B=2, Hq=32, Hkv=8, N=N, d=128, dtype="bf16", seed=40 + i, seqlens=sl)
        q, k, v, s = upload(inp)
        cases.append((q, k, v, s, chunk, ta.decode(q, k, v, s, chunk=chunk)))
    torch.cuda.synchronize()
    log(f"concurrent: 3 threads x 20 calls over {len(cases)} shapes")
    errors = []

    def worker(tid):
        try:
            stream = torch.cuda.Stream()
            with torch.cuda.stream(stream):
                for it in range(20):
                    q, k, v, s, chunk, (ref_o, ref_l) = cases[(tid + it) % len(cases)]
                    out, lse = ta.decode(q, k, v, s, chunk=chunk, stream=stream)
                    stream.synchronize()
                    if not (torch.equal(out, ref_o) and torch.equal(lse, ref_l)):
                        errors.append(f"thread {tid}, call {it}: result differs")
        except Exception as e:  # reported below, in the main thread
            errors.append(f"thread {tid}: {e!r}")

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(3)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=60)
    assert not any(t.is_alive() for t in threads), "a worker thread did not finish"
    assert not errors, errors


def test_concurrent_threads_on_one_stream():
    # Several host threads enqueue decode steps on one shared stream without waiting
    # in between, over shapes that grow (so the stream's workspace is replaced while
    # other threads' steps are queued on it). Each call holds the workspace until its
    # last launch, so every step's merge reads its own partial states: every result
    # must equal the single-thread one bit for bit.
    import threading
    cases = []
    for i, (B, N, chunk) in enumerate([(1, 3000, 512), (2, 12000, 256), (2, 30000, 128), (4, 30000, 64)]):
        inp = W.random_decode(B=B, Hq=32, Hkv=8, N=N, d=128, dtype="bf16", seed=90 + i,
                              seqlens=[N - 7 * b for b in range(B)])
        q, k, v, s = upload(inp)
        cases.append((q, k, v, s, chunk, ta.decode(q, k, v, s, chunk=chunk)))
    torch.cuda.synchronize()
    shared = torch.cuda.Stream()  # a fresh stream: its workspace starts empty and grows
    n_threads, n_calls = 3, 24
    log(f"one stream: {n_threads} threads x {n_calls} calls over {len(cases)} growing shapes")
    results = [[] for _ in range(n_threads)]
    errors = []
    start = threading.Barrier(n_threads)

    def worker(tid):
        try:
            start.wait()
            for it in range(n_calls):
                ci = min(len(cases) - 1, (it * len(cases)) // n_calls + (tid + it) % 2)
                q, k, v, s, chunk, _ = cases[ci]
                results[tid].append((ci, ta.decode(q, k, v, s, chunk=chunk, stream=shared)))
        except Exception as e:  # reported below, in the main thread
            errors.append(f"thread {tid}: {e!r}")

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(n_threads)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a worker thread did not finish"
    shared.synchronize()
    assert not errors, errors
    for tid in range(n_threads):
        for it, (ci, (out, lse)) in enumerate(results[tid]):
            ref_o, ref_l = cases[ci][5]
            assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), f"thread {tid}, call {it} (shape {ci}) differs"


def test_seqlens_none_and_lse_none_paths():
    inp = W.random_decode(B=1, Hq=8, Hkv=2, N=1000, d=64, dtype="bf16", seed=14)
    q, k, v, _ = upload(inp)
    out, lse = ta.decode(q, k, v, None, chunk=128)
    torch.cuda.synchronize()
    ro, rl = oracle.decode(inp.q, inp.k, inp.v, None)
    assert_close(out.cpu().numpy(), lse.cpu().numpy(), ro, rl, "bf16", what="no seqlens")


# ---------------------------------------------------------------- workload sizes

@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["gqa8b_128k", "gqa8b_1m", "gqa8b_512k_b4_peaked", "gqa8b_ragged_b32"])
def test_workload_sized_all_rows(name):
    # every (sequence, head) row of each large workload, element by element, in the
    # launch configuration the benchmark times
    wl = W.WORKLOADS[name]
    log(f"workload {name}: generating inputs")
    inp = W.make_decode_inputs(wl, 1)
    q, k, v, sl = upload(inp)
    sl = sl if wl.ragged is not None else None  # as the benchmark passes them
    log(f"workload {name}: on device, running decode (chunk {wl.chunk})")
    out, lse = ta.decode(q, k, v, sl, chunk=wl.chunk)
    torch.cuda.synchronize()
    out, lse = out.cpu().numpy().reshape(-1, wl.d), lse.cpu().numpy().reshape(-1)
    del q, k, v
    torch.cuda.empty_cache()
    log(f"workload {name}: oracle on all {wl.B * wl.Hq} rows")
    ro, rl = oracle.decode(inp.q, inp.k, inp.v, inp.seqlens)
    err, lerr = assert_close(out, lse, ro.reshape(-1, wl.d), rl.reshape(-1), wl.dtype, what=name)
    log(f"workload {name}: max abs out err {err:.2e}, max rel lse err {lerr:.2e}")


@pytest.mark.timeout(300)
def test_combine_workload_full_size():
    # the standalone merge workload in full: 32 x 32 heads x 64 fp32 states, d = 128,
    # at the fp32 bar; then the same states with about a tenth of them empty
    cw = W.COMBINE_WORKLOADS["combine_64x128"]
    ci = W.make_combine_inputs(cw, 1)
    po = torch.from_numpy(ci.partial_o).cuda()
    pl_np = ci.partial_lse.copy()
    for label in ("as drawn", "with empty states"):
        if label == "with empty states":
            rng = np.random.default_rng(5)
            pl_np[rng.random(pl_np.shape) < 0.1] = -np.inf
            pl_np[3, 7, :] = -np.inf  # one row with no state at all
        pl = torch.from_numpy(pl_np).cuda()
        log(f"combine_64x128 {label}")
        out, lse = ta.combine(po, pl)
        torch.cuda.synchronize()
        ro, rl = oracle.combine(ci.partial_o, pl_np)
        assert_close(out.cpu().numpy(), lse.cpu().numpy(), ro, rl, "f32", what=f"combine_64x128 {label}")


def _merged_by_separate_pass(q, k, v, sl, chunk):
    po, pl = ta.partial(q, k, v, sl, chunk=chunk)
    return ta.combine(po, pl)


@pytest.mark.parametrize("N,chunk", [(2000, 300), (8000, 100), (8000, 63), (3000, 1)])
def test_decode_equals_combine_of_partials(N, chunk):
    # P = 7, 80 and 127 merge in one pass; P = 3000 in several passes
    inp = W.random_decode(B=3, Hq=8, Hkv=2, N=N, d=128, dtype="bf16", seed=N + chunk,
                          seqlens=[N, N // 3, 0])
    q, k, v, sl = upload(inp)
    log(f"decode vs partial + combine: N={N} chunk={chunk}")
    for _ in range(3):  # repeated launches reuse the stream's workspace
        out, lse = ta.decode(q, k, v, sl, chunk=chunk)
        ref_o, ref_l = _merged_by_separate_pass(q, k, v, sl, chunk)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l)
    ro, rl = oracle.decode(inp.q, inp.k, inp.v, inp.seqlens)
    assert_close(out.cpu().numpy(), lse.cpu().numpy(), ro, rl, "bf16", what=f"N={N} chunk={chunk}")


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64)])
def test_partial_of_an_empty_cache(dtype, d):
    # N = 0: slot 0 of every row holds the empty state, and merging it gives what
    # ta_decode gives (out = 0, lse = -inf), bit for bit
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    q = torch.randn(2, 8, d, device="cuda").to(tdt)
    # tensors with no elements have a NULL data pointer, which the library accepts
    k = torch.empty(2, 2, 0, d, dtype=tdt, device="cuda")
    v = torch.empty(2, 2, 0, d, dtype=tdt, device="cuda")
    po = torch.full((2, 8, 1, d), float("nan"), device="cuda")
    pl = torch.full((2, 8, 1), float("nan"), device="cuda")
    ta.partial(q, k, v, None, chunk=64, partial_o=po, partial_lse=pl)
    po2, pl2 = ta.partial(q, k, v, None, chunk=64)  # the binding allocates the one slot
    out, lse = ta.decode(q, k, v, None, chunk=64)
    co, cl = ta.combine(po, pl)
    torch.cuda.synchronize()
    for a, b in ((po, pl), (po2, pl2)):
        assert torch.equal(a, torch.zeros_like(a)) and bool(torch.isneginf(b).all())
    assert torch.equal(out, torch.zeros_like(out)) and bool(torch.isneginf(lse).all())
    assert torch.equal(co, out) and torch.equal(cl, lse)


# ta_decode (and ta_decode_noalloc) against ta_partial + ta_combine, bit for bit, over
# grids of one round and of several, 1 to 128 states per row, empty rows included;
# repeated calls reuse the same workspace.
DECODE_VS_SEPARATE_CASES = [
    # (B, N, chunk, seqlens or None): P = 1, 2, 3, 8, 64, 65, 127, 128
    (2, 300, 512, None), (2, 600, 300, [600, 1]), (3, 700, 256, [700, 0, 513]), (2, 4096, 512, None),
    (2, 8192, 128, [8192, 4000]), (1, 8320, 128, None), (2, 16256, 128, [16256, 129]), (1, 16384, 128, None),
]


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("f32", 128), ("f32", 64)])
@pytest.mark.parametrize("Hq,Hkv", [(32, 8), (8, 4), (4, 4)])
@pytest.mark.parametrize("case", DECODE_VS_SEPARATE_CASES, ids=lambda c: f"B{c[0]}N{c[1]}c{c[2]}{'r' if c[3] else ''}")
def test_decode_equals_separate_merge_over_shapes(case, Hq, Hkv, dtype, d):
    B, N, chunk, sl = case
    inp = W.random_decode(B=B, Hq=Hq, Hkv=Hkv, N=N, d=d, dtype=dtype, seed=N + chunk + Hq, seqlens=sl)
    q, k, v, s = upload(inp)
    s = s if sl is not None else None
    log(f"decode vs separate merge: B={B} Hq={Hq} Hkv={Hkv} N={N} d={d} {dtype} chunk={chunk} seqlens={sl}")
    ref_o, ref_l = _merged_by_separate_pass(q, k, v, s, chunk)
    for rep in range(3):
        out, lse = ta.decode(q, k, v, s, chunk=chunk)
        na_o, na_l = ta.decode_noalloc(q, k, v, s, chunk=chunk)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), f"repeat {rep}: decode differs"
        assert torch.equal(na_o, ref_o) and torch.equal(na_l, ref_l), f"repeat {rep}: decode_noalloc differs"
    ro, rl = oracle.decode(inp.q, inp.k, inp.v, inp.seqlens)
    assert_close(out.cpu().numpy(), lse.cpu().numpy(), ro, rl, dtype, what="decode vs separate merge")


@pytest.mark.parametrize("N,chunk", [(262144, 4096), (524288, 8192)])
def test_several_chunks_kernel_decode_equals_separate_merge(N, chunk):
    # one workgroup per CU streaming several chunks (2 and 2 per workgroup here)
    inp = W.random_decode(B=1, Hq=32, Hkv=8, N=N, d=128, dtype="bf16", seed=N // chunk)
    q, k, v, _ = upload(inp)
    log(f"several chunks per workgroup: N={N} chunk={chunk}")
    ref_o, ref_l = _merged_by_separate_pass(q, k, v, None, chunk)
    for _ in range(2):
        out, lse = ta.decode(q, k, v, None, chunk=chunk)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l)
    ro, rl = oracle.decode(inp.q, inp.k, inp.v, inp.seqlens)
    assert_close(out.cpu().numpy(), lse.cpu().numpy(), ro, rl, "bf16", what=f"N={N}")


def test_shapes_alternate_on_one_stream_and_a_second_stream():
    # different head-group counts and partial counts reuse one stream's workspace; a
    # second stream gets its own
    cases = [W.random_decode(B=2, Hq=32, Hkv=8, N=5000, d=128, dtype="bf16", seed=s, seqlens=[5000, 77])
             for s in (1, 2)] + [W.random_decode(B=5, Hq=4, Hkv=4, N=900, d=64, dtype="f32", seed=3,
                                                  seqlens=[900, 1, 450, 0, 899])]
    side = torch.cuda.Stream()
    for rep in range(2):
        for i, inp in enumerate(cases):
            q, k, v, sl = upload(inp)
            chunk = [256, 1024, 64][i]
            stream = side if rep == 1 else None
            if stream is not None:
                stream.wait_stream(torch.cuda.current_stream())
                with torch.cuda.stream(stream):
                    out, lse = ta.decode(q, k, v, sl, chunk=chunk)
                torch.cuda.current_stream().wait_stream(stream)
            else:
                out, lse = ta.decode(q, k, v, sl, chunk=chunk)
            torch.cuda.synchronize()
            ro, rl = oracle.decode(inp.q, inp.k, inp.v, inp.seqlens)
            dtype = "bf16" if inp.q.dtype == np.uint16 else "f32"
            assert_close(out.cpu().numpy(), lse.cpu().numpy(), ro, rl, dtype, what=f"case {i} rep {rep}")


@pytest.mark.parametrize("chunk", [512, 16])
def test_graph_capture_replays_match_eager(chunk):
    # under capture the library allocates its workspace inside the captured work; chunk 16
    # gives 313 partial states per row, so the merge also runs in several passes there
    inp = W.random_decode(B=2, Hq=8, Hkv=2, N=5000, d=128, dtype="bf16", seed=40, seqlens=[5000, 2222])
    other = W.random_decode(B=2, Hq=8, Hkv=2, N=5000, d=128, dtype="bf16", seed=41, seqlens=[4000, 5000])
    q, k, v, sl = upload(inp)
    q2, k2, v2, sl2 = upload(other)
    ref_o, ref_l = ta.decode(q, k, v, sl, chunk=chunk)
    ref2_o, ref2_l = ta.decode(q2, k2, v2, sl2, chunk=chunk)
    out = torch.empty_like(ref_o)
    lse = torch.empty_like(ref_l)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        ta.decode(q, k, v, sl, chunk=chunk, out=out, lse=lse)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    log(f"capturing decode, chunk {chunk}")
    with torch.cuda.graph(g):
        ta.decode(q, k, v, sl, chunk=chunk, out=out, lse=lse)
    for rep in range(4):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), f"replay {rep}"
        # eager work on the same stream between replays
        o2, l2 = ta.decode(q2, k2, v2, sl2, chunk=chunk)
        torch.cuda.synchronize()
        assert torch.equal(o2, ref2_o) and torch.equal(l2, ref2_l)
    del g
    torch.cuda.synchronize()


def test_out_of_range_seqlens_are_clamped():
    # lengths outside [0, N] are clamped to it (the header's contract)
    inp = W.random_decode(B=3, Hq=8, Hkv=2, N=700, d=128, dtype="bf16", seed=50, seqlens=[700, 0, 300])
    q, k, v, _ = upload(inp)
    bad = torch.tensor([700 + 1000, -5, 300], dtype=torch.int32, device="cuda")
    out, lse = ta.decode(q, k, v, bad, chunk=128)
    torch.cuda.synchronize()
    ro, rl = oracle.decode(inp.q, inp.k, inp.v, inp.seqlens)
    assert_close(out.cpu().numpy(), lse.cpu().numpy(), ro, rl, "bf16", what="clamped seqlens")


# ---------------------------------------------------------------- strides, determinism, capture

def test_combine_reads_strided_partials():
    # states stored leaf-major [P, B, H, d] and passed as a permuted [B, H, P, d] view
    P, B, H, d = 200, 2, 3, 128
    po_np, pl_np = combine_inputs_with_empties(B, H, P, d, 61)
    po_lm = dev_tensor(np.ascontiguousarray(po_np.transpose(2, 0, 1, 3)))   # [P, B, H, d]
    pl_lm = dev_tensor(np.ascontiguousarray(pl_np.transpose(2, 0, 1)))      # [P, B, H]
    po_v, pl_v = po_lm.permute(1, 2, 0, 3), pl_lm.permute(1, 2, 0)
    assert not po_v.is_contiguous()
    for arity in (None, 4, "chain"):
        out, lse = ta.combine(po_v, pl_v, arity=arity)
        torch.cuda.synchronize()
        ro, rl = oracle.combine(po_np, pl_np)
        assert_close(out.cpu().numpy(), lse.cpu().numpy(), ro, rl, "f32", what=f"strided combine {arity}")


def test_decode_with_strided_q_and_output_slices():
    inp = W.random_decode(B=2, Hq=8, Hkv=2, N=1200, d=128, dtype="bf16", seed=62, seqlens=[1200, 555])
    q, k, v, sl = upload(inp)
    # q inside a wider buffer ([B, Hq, 2d], every other d-block), out and lse inside bigger tensors
    wide = torch.zeros(2, 8, 256, dtype=torch.bfloat16, device="cuda")
    wide[:, :, 128:] = q
    q_view = wide[:, :, 128:]
    big_out = torch.full((2, 10, 128), 5.0, device="cuda")
    big_lse = torch.full((2, 10, 3), 5.0, device="cuda")
    out_view, lse_view = big_out[:, 1:9], big_lse[:, 1:9, 1]  # lse with a token stride of 3
    ta.decode(q_view, k, v, sl, chunk=256, out=out_view, lse=lse_view)
    torch.cuda.synchronize()
    ro, rl = oracle.decode(inp.q, inp.k, inp.v, inp.seqlens)
    assert_close(out_view.cpu().numpy(), lse_view.cpu().numpy(), ro, rl, "bf16", what="strided q / output views")
    # nothing outside the views was written
    assert torch.all(big_out[:, 0] == 5.0) and torch.all(big_out[:, 9] == 5.0)
    assert torch.all(big_lse[:, :, 0] == 5.0) and torch.all(big_lse[:, :, 2] == 5.0)
    assert torch.all(big_lse[:, 0, 1] == 5.0) and torch.all(big_lse[:, 9, 1] == 5.0)


@pytest.mark.parametrize("arity", [3, 8, "chain"])
def test_merge_variants_bitwise_deterministic(arity):
    po_np, pl_np = combine_inputs_with_empties(4, 8, 700, 128, 63)
    po, pl = dev_tensor(po_np), dev_tensor(pl_np)
    a = ta.combine(po, pl, arity=arity)
    b = ta.combine(po, pl, arity=arity)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_graph_capture_of_multipass_arity_merge():
    # 5000 leaves at arity 4 (256 per launch) take two passes through workspace
    # allocated inside the capture; replays must match the eager result every time
    po_np, pl_np = combine_inputs_with_empties(2, 3, 5000, 64, 64)
    po, pl = dev_tensor(po_np), dev_tensor(pl_np)
    ref_o, ref_l = ta.combine(po, pl, arity=4)
    out, lse = torch.empty_like(ref_o), torch.empty_like(ref_l)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        ta.combine(po, pl, out=out, lse=lse, arity=4)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    log("capturing a two-pass arity-4 merge")
    with torch.cuda.graph(g):
        ta.combine(po, pl, out=out, lse=lse, arity=4)
    for rep in range(3):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), f"replay {rep}"
        o2, _ = ta.combine(po[:, :, :77].contiguous(), pl[:, :, :77].contiguous(), arity=4)  # eager work between
        torch.cuda.synchronize()
    del g
    torch.cuda.synchronize()


def test_binding_raises_the_library_code_and_message():
    inp = W.random_decode(B=1, Hq=8, Hkv=2, N=256, d=128, dtype="bf16", seed=70)
    q, k, v, _ = upload(inp)
    with pytest.raises(ValueError):  # host tensors never reach the library
        ta.decode(q.cpu(), k, v, None, chunk=64)
    with pytest.raises(ta.TreeAttnError) as e:
        ta.decode(q, k, v, None, chunk=0)
    assert e.value.code == ta.TA_ERR_ARG and "chunk" in str(e.value)
    with pytest.raises(ta.TreeAttnError) as e:
        ta.decode(q, k[:, :, :, :64], v, None, chunk=64)  # k and v shapes differ
    assert e.value.code == ta.TA_ERR_SHAPE
    po = torch.zeros(1, 8, 4, 128, device="cuda")
    pl = torch.zeros(1, 8, 4, device="cuda")
    with pytest.raises(ta.TreeAttnError) as e:
        ta.combine(po, pl, arity=17)
    assert e.value.code == ta.TA_ERR_ARG and "arity" in str(e.value)
    # a failed call leaves the stream usable
    out, lse = ta.decode(q, k, v, None, chunk=64)
    torch.cuda.synchronize()
    ro, rl = oracle.decode(inp.q, inp.k, inp.v, inp.seqlens)
    assert_close(out.cpu().numpy(), lse.cpu().numpy(), ro, rl, "bf16", what="after errors")


def test_sharded_decode_then_combine_is_the_full_decode():
    # The multi-GPU split on one device, with public calls only: each "shard" decodes
    # its own token range of the cache (a strided view, its own lengths), and one
    # ta_combine over the shard outputs, as leaves (o_r, lse_r), gives the full decode.
    G, N = 4, 4096
    inp = W.random_decode(B=3, Hq=32, Hkv=8, N=N, d=128, dtype="bf16", seed=71, seqlens=[4096, 2500, 700])
    q, k, v, sl = upload(inp)
    n = N // G
    outs, lses = [], []
    for r in range(G):
        lens = torch.clamp(sl - r * n, 0, n).to(torch.int32)  # shard 3 of sequence 3 is empty
        o, l = ta.decode(q, k[:, :, r * n:(r + 1) * n], v[:, :, r * n:(r + 1) * n], lens, chunk=256)
        outs.append(o)
        lses.append(l)
    po = torch.stack(outs, dim=2)   # [B, Hq, G, d]
    pl = torch.stack(lses, dim=2)   # [B, Hq, G]
    out, lse = ta.combine(po, pl)
    torch.cuda.synchronize()
    ro, rl = oracle.decode(inp.q, inp.k, inp.v, inp.seqlens)
    assert_close(out.cpu().numpy(), lse.cpu().numpy(), ro, rl, "bf16", what="shards + combine")
    full_o, full_l = ta.decode(q, k, v, sl, chunk=256)
    torch.cuda.synchronize()
    assert (out - full_o).abs().max().item() < 1e-5 and (lse - full_l).abs().max().item() < 1e-4


@pytest.mark.parametrize("B,Hq,Hkv,N,chunk", [
    (65535, 1, 1, 24, 8),      # the largest batch: the partial grid's z and the merge grid's y at 65535
    (1, 65535, 65535, 8, 4),   # the most query heads: 65535 head groups of one head each
    (2, 2, 1, 4096 * 8 + 3, 4096),  # 9 chunks of 4096 and a 3-token tail
])
def test_grid_limits(B, Hq, Hkv, N, chunk):
    inp = W.random_decode(B=B, Hq=Hq, Hkv=Hkv, N=N, d=64, dtype="bf16", seed=80,
                          seqlens=[N - (b % 5) for b in range(B)])
    log(f"grid limits: B={B} Hq={Hq} Hkv={Hkv} N={N} chunk={chunk}")
    q, k, v, sl = upload(inp)
    out, lse = ta.decode(q, k, v, sl, chunk=chunk)
    torch.cuda.synchronize()
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    rows = np.unique(np.concatenate([np.arange(0, 64), np.arange(B * Hq - 64, B * Hq),
                                     np.random.default_rng(1).choice(B * Hq, 64)]))
    rows = rows[(rows >= 0) & (rows < B * Hq)]
    ro, rl = oracle.decode(inp.q, inp.k, inp.v, inp.seqlens, rows=rows)
    assert_close(out.reshape(-1, 64)[rows], lse.reshape(-1)[rows], ro, rl, "bf16", what=f"grid limits B={B} Hq={Hq}")


def test_prepared_decode_reads_its_buffers_at_each_call():
    a = W.random_decode(B=2, Hq=8, Hkv=2, N=900, d=128, dtype="bf16", seed=90, seqlens=[900, 333])
    b = W.random_decode(B=2, Hq=8, Hkv=2, N=900, d=128, dtype="bf16", seed=91, seqlens=[500, 900])
    q, k, v, sl = upload(a)
    qb, kb, vb, slb = upload(b)
    step = ta.PreparedDecode(q, k, v, sl, chunk=128)
    out, lse = step()
    ref = ta.decode(q, k, v, sl, chunk=128)
    torch.cuda.synchronize()
    assert torch.equal(out, ref[0]) and torch.equal(lse, ref[1])
    # refill the same buffers in place: the next call sees the new contents
    q.copy_(qb); k.copy_(kb); v.copy_(vb); sl.copy_(slb)
    out, lse = step()
    torch.cuda.synchronize()
    ro, rl = oracle.decode(b.q, b.k, b.v, b.seqlens)
    assert_close(out.cpu().numpy(), lse.cpu().numpy(), ro, rl, "bf16", what="prepared decode, refilled")


def _random_configs(n, seed):
    rng = np.random.default_rng(seed)
    cfgs = []
    for i in range(n):
        d = int(rng.choice([64, 128]))
        dtype = str(rng.choice(["bf16", "f32"]))
        Hkv = int(rng.choice([1, 2, 4, 8]))
        G = int(rng.choice([1, 2, 3, 4, 5, 8]))
        B = int(rng.integers(1, 9))
        N = int(rng.integers(1, 6000))
        chunk = int(rng.choice([1, 7, 16, 64, 128, 300, 512, 1024, 4096]))
        if N // chunk > 3000:  # keep every case small enough for the oracle
            chunk = max(chunk, N // 3000 + 1)
        lens = [int(x) for x in rng.integers(0, N + 1, size=B)]
        if rng.random() < 0.5:
            lens = None
        cfgs.append(dict(B=B, Hq=Hkv * G, Hkv=Hkv, N=N, d=d, dtype=dtype, chunk=chunk, seqlens=lens, seed=1000 + i))
    return cfgs


@pytest.mark.parametrize("cfg", _random_configs(48, 2024), ids=lambda c: f"B{c['B']}H{c['Hq']}/{c['Hkv']}N{c['N']}d{c['d']}{c['dtype']}c{c['chunk']}{'r' if c['seqlens'] else ''}")
def test_random_shapes_against_oracle(cfg):
    # a seeded mix of batch, GQA ratio, length, head dim, dtype, chunk and ragged
    # lengths: small and large grids (4- and 8-wave workgroups), rotated chunk
    # orders, multi-pass merges
    c = dict(cfg)
    chunk, sl, seed = c.pop("chunk"), c.pop("seqlens"), c.pop("seed")
    inp = W.random_decode(**c, seed=seed, seqlens=sl)
    log(f"random shape {cfg}")
    q, k, v, sl_d = upload(inp)
    out, lse = ta.decode(q, k, v, sl_d if sl is not None else None, chunk=chunk)
    torch.cuda.synchronize()
    ro, rl = oracle.decode(inp.q, inp.k, inp.v, inp.seqlens)
    assert_close(out.cpu().numpy(), lse.cpu().numpy(), ro, rl, c["dtype"], what=f"random {cfg}")


def test_suggest_chunk_reads_the_device():
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for n in (8192, 131072, 1 << 20):
        assert ta.suggest_chunk(1, 32, 8, n) == ta.suggest_chunk(1, 32, 8, n, compute_units=cus)


@pytest.mark.parametrize("B,per_cu,dtype,d,Hkv", [
    (1, 4, "bf16", 128, 8), (1, 8, "bf16", 128, 8), (2, 4, "bf16", 128, 8), (1, 4, "bf16", 64, 8),
    (1, 5, "f32", 128, 8), (2, 4, "f32", 64, 8), (1, 2, "bf16", 128, 8), (3, 6, "bf16", 128, 8),
    (1, 8, "bf16", 128, 4), (1, 4, "f32", 128, 4),  # 8 query heads per workgroup: per-chunk kernel either way
    (4, 16, "bf16", 128, 8), (1, 16, "bf16", 64, 8),  # 16 chunks per workgroup
])
def test_several_chunks_per_workgroup_are_bitwise_the_per_chunk_states(B, per_cu, dtype, d, Hkv):
    # Without seqlens, rows of whole chunks in a grid of exactly 4 to 16 rounds of CUs
    # go to the kernel that streams several chunks per workgroup (not with 8 query heads
    # per workgroup, which keep the per-chunk grid); full-length seqlens take the
    # per-chunk kernel over the same tokens. Every state, and ta_decode's result, must
    # be the same bits. 2 rounds, and B = 3 at 6 rounds (64 chunks per row, no multiple
    # of 6), stay on the per-chunk kernel.
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    Hq, chunk = 32, 2048
    groups = Hq // min(8, Hq // Hkv)  # workgroups per chunk of a sequence (Hq / Hkv is 4 or 8 here)
    if (per_cu * cus) % (groups * B):
        pytest.skip(f"{per_cu} rounds of {cus} CUs is no whole number of chunks per row")
    n_chunks = per_cu * cus // (groups * B)
    N = n_chunks * chunk
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    gen = torch.Generator(device="cuda").manual_seed(B * 100 + per_cu * 10 + d)
    q = torch.randn(B, Hq, d, generator=gen, device="cuda").to(tdt)
    k = torch.randn(B, Hkv, N, d, generator=gen, device="cuda").to(tdt)
    v = torch.randn(B, Hkv, N, d, generator=gen, device="cuda").to(tdt)
    full = torch.full((B,), N, dtype=torch.int32, device="cuda")
    log(f"chunks per workgroup: B={B} Hkv={Hkv} {dtype} d={d} N={N} ({n_chunks} chunks per row, {per_cu} rounds of {cus} CUs)")
    a = ta.partial(q, k, v, None, chunk=chunk)
    b = ta.partial(q, k, v, full, chunk=chunk)
    torch.cuda.synchronize()
    assert torch.isfinite(a[0]).all() and torch.isfinite(a[1]).all()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    c = ta.decode(q, k, v, None, chunk=chunk)
    e = ta.decode(q, k, v, full, chunk=chunk)
    torch.cuda.synchronize()
    assert torch.equal(c[0], e[0]) and torch.equal(c[1], e[1])
