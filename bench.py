#!/usr/bin/env python3
"""Decode-attention benchmark on one MI355X.

One step = one ta_decode call: the split-KV partial-state kernel over the whole
KV cache, then the tree merge, for every sequence and query head of the
workload. Default workload: the Llama-3.1-8B attention shape (32 query heads,
8 KV heads, d = 128), bf16, batch 1, 131072-token context, chunk 2048 (64
partial states, a 6-level tree), seeded synthetic N(0,1) inputs.

Timing: W untimed warm-up steps, then exactly K steps between two device
synchronisations, bracketed by HIP events on the stream the kernels run on.
The step inputs rotate over several resident copies of the cache (at least
2 GiB in total, far above the 256 MB last-level cache), so every step streams
its K/V from HBM. The dominant kernel (partial states) is also timed alone with
events over K launches, for the roofline figure. The CPU oracle is timed on the
same host over a bounded sample, as a baseline only.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode-attn µs/step + achieved HBM GB/s (% peak), 8B-GQA bf16 128k ctx"
HBM_PEAK_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_partial_gqa8b_128k.json")
PARTIAL_SRC = os.path.join(ROOT, "softmax_tree_reduction_amd", "csrc", "partial.hip")


def algorithmic_bytes(wl, seqlens) -> int:
    """K + V rows of every valid token, q, out (f32) and lse (f32)."""
    es = 2 if wl.dtype == "bf16" else 4
    kv = 2 * int(sum(int(n) for n in seqlens)) * wl.Hkv * wl.d * es
    return kv + wl.B * wl.Hq * wl.d * es + wl.B * wl.Hq * wl.d * 4 + wl.B * wl.Hq * 4


def file_sha256(path: str) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def measured_traffic(wl_name: str):
    """HBM bytes per partial-kernel launch from the committed rocprofv3 counter runs,
    or None when they are missing or were taken on a different kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("workload") != wl_name or t.get("partial_hip_sha256") != file_sha256(PARTIAL_SRC):
        return None
    return t.get("bytes_per_launch")


def host_cpu() -> dict:
    """The host's CPU model (from /proc/cpuinfo, as lscpu reports it) and the logical
    CPUs the machine has and this process may use."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = None
    return {"model": model, "logical_cpus": os.cpu_count(), "usable_cpus": usable}


def cpu_baseline(inp, wl, budget_s: float):
    """The oracle, untouched, on the full step (all rows), repeated within a time budget."""
    import oracle
    oracle.build()
    t0 = time.perf_counter()
    oracle.decode(inp.q, inp.k, inp.v, inp.seqlens)
    first = time.perf_counter() - t0
    reps = max(1, min(5, int(budget_s / max(first, 1e-3))))
    times = [first]
    for _ in range(reps - 1):
        t0 = time.perf_counter()
        oracle.decode(inp.q, inp.k, inp.v, inp.seqlens)
        times.append(time.perf_counter() - t0)
    times.sort()
    med = times[len(times) // 2]
    step_bytes = algorithmic_bytes(wl, inp.seqlens)
    gbs = step_bytes / med / 1e9
    cores = oracle.num_threads()
    # the same step on one thread (one run; the rows are independent, so the result is the same)
    oracle.set_num_threads(1)
    try:
        t0 = time.perf_counter()
        oracle.decode(inp.q, inp.k, inp.v, inp.seqlens)
        one = time.perf_counter() - t0
    finally:
        oracle.set_num_threads(cores)
    return {"value": round(gbs, 3), "unit": "GB/s", "cores": cores, "kind": "oracle", "cpu": host_cpu(),
            "sample": f"the full step of {wl.name} (all {wl.B * wl.Hq} query rows, {int(sum(inp.seqlens))} tokens "
                      f"per KV head), float64 two-pass definition, median of {len(times)} runs, "
                      f"{med * 1e3:.1f} ms per step",
            "single_thread": {"value": round(step_bytes / one / 1e9, 3), "unit": "GB/s",
                              "ms_per_step": round(one * 1e3, 1)}}


def settle_and_read_ceiling(ta, torch, dev, stream, settle_ms: float):
    """Streams a 1 GiB buffer (several times the caches) with ta_stream_read for
    `settle_ms` of device time, then times 20 more reads: the practical read ceiling.
    The device reaches its steady speed only after some tens of ms of sustained load,
    so this runs before anything is timed. Returns (settled ms, reads, GB/s)."""
    probe = torch.empty(2**30, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    settled_ms, reads = 0.0, 0
    while True:
        ev0.record(stream)
        for _ in range(3 if reads == 0 else 50):
            ta.stream_read(probe, sink)
            reads += 1
        ev1.record(stream)
        torch.cuda.synchronize()
        settled_ms += ev0.elapsed_time(ev1)
        if settled_ms >= settle_ms:
            break
    ev0.record(stream)
    for _ in range(20):
        ta.stream_read(probe, sink)
    ev1.record(stream)
    torch.cuda.synchronize()
    ceiling = probe.numel() / (ev0.elapsed_time(ev1) / 20 * 1e-3) / 1e9
    del probe
    return settled_ms, reads, ceiling


def bench_combine(args, dev) -> int:
    """ta_combine (or ta_combine_k with --arity K) alone on the combine workload:
    one GPU's share of a 64-shard merge."""
    import numpy as np
    import torch

    import oracle
    import softmax_tree_reduction_amd as ta
    import workloads as W

    cw = W.COMBINE_WORKLOADS["combine_64x128"]
    if args.n_parts:  # the same rows with another number of states each
        cw = dataclasses.replace(cw, name=f"combine_{args.n_parts}x128", n_parts=args.n_parts)
    ci = W.make_combine_inputs(cw, args.seed)
    nbytes = (ci.partial_o.nbytes + ci.partial_lse.nbytes) + cw.B * cw.H * (cw.d + 1) * 4
    copies = max(1, math.ceil(args.min_rotation_bytes / nbytes))
    pos = [torch.from_numpy(ci.partial_o).to(dev) for _ in range(copies)]
    pls = [torch.from_numpy(ci.partial_lse).to(dev) for _ in range(copies)]
    out = torch.empty(cw.B, cw.H, cw.d, dtype=torch.float32, device=dev)
    lse = torch.empty(cw.B, cw.H, dtype=torch.float32, device=dev)
    ta.combine(pos[0], pls[0], out=out, lse=lse, arity=args.arity)
    torch.cuda.synchronize()
    ro, rl = oracle.combine(ci.partial_o, ci.partial_lse)
    err = float(np.abs(out.cpu().numpy() - ro).max())
    lerr = float((np.abs(lse.cpu().numpy() - rl) / np.maximum(1.0, np.abs(rl))).max())
    # the chain's longest rounding path has P - 1 merges: recursive-summation bound
    tol = 1e-5 if args.arity != "chain" else max(1e-5, 4 * (cw.n_parts - 1) * 2.0 ** -24 * float(np.abs(ci.partial_o).max()))
    if not (err <= tol and lerr <= 1e-4):
        print(f"bench: combine parity failed ({err}, {lerr})", file=sys.stderr)
        return 1
    stream = torch.cuda.current_stream(dev)
    settled_ms, _, _ = settle_and_read_ceiling(ta, torch, dev, stream, args.settle_ms)
    for i in range(args.warmup):
        ta.combine(pos[i % copies], pls[i % copies], out=out, lse=lse, arity=args.arity)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for i in range(args.steps):
        ta.combine(pos[i % copies], pls[i % copies], out=out, lse=lse, arity=args.arity)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    # the same calls replayed from a captured graph: device time without the binding's
    # per-call host cost (which is about as long as the kernel)
    side = torch.cuda.Stream(dev)
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        ta.combine(pos[0], pls[0], out=out, lse=lse, arity=args.arity)
    stream.wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(args.steps):
            ta.combine(pos[i % copies], pls[i % copies], out=out, lse=lse, arity=args.arity)
    graph.replay()
    torch.cuda.synchronize()
    ev0.record(stream)
    graph.replay()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms_graph = ev0.elapsed_time(ev1) / args.steps
    del graph
    kernel = {None: "ta_combine", "chain": "ta_combine_chain"}.get(args.arity, "ta_combine_k")
    print(json.dumps({"mode": "combine", "workload": cw.name, "arity": args.arity or 2,
                      "kernel": kernel, "us_per_call": round(ms * 1e3, 2),
                      "us_per_call_graph": round(ms_graph * 1e3, 2),
                      "bytes_per_call": nbytes, "GB_per_s": round(nbytes / (ms * 1e-3) / 1e9, 1),
                      "GB_per_s_graph": round(nbytes / (ms_graph * 1e-3) / 1e9, 1),
                      "settle_ms": round(settled_ms, 1),
                      "rows": cw.B * cw.H, "n_parts": cw.n_parts, "copies": copies,
                      "max_abs_out_err": err, "max_rel_lse_err": lerr}))
    return 0


def bench_floor(args, dev) -> int:
    """Floors of the merge stage. Prints one JSON line with, in µs per call:
    - empty_launch: ta_stream_read over 16 bytes (one workgroup, one load), replayed
      from a captured graph: what a launch costs with no work;
    - read_combine_bytes: ta_stream_read over the merge workload's 34.3 MB, rotated
      over resident copies as --mode combine rotates its inputs (graph replay);
    - combine: ta_combine on the merge workload (32 x 32 rows of 64 states), same way;
    - on the 128k decode workload, eager loops over the cache rotation: ta_partial
      alone, ta_partial followed by the empty launch, ta_partial followed by ta_combine
      of its states, and ta_decode. The differences to ta_partial alone are what a
      dependent second launch, and the merge, add to a decode step."""
    import numpy as np
    import torch

    import softmax_tree_reduction_amd as ta
    import workloads as W

    stream = torch.cuda.current_stream(dev)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def graph_us(fn, reps):
        side = torch.cuda.Stream(dev)
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            fn(0)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(reps):
                fn(i)
        graph.replay()
        torch.cuda.synchronize()
        ev0.record(stream)
        graph.replay()
        ev1.record(stream)
        torch.cuda.synchronize()
        del graph
        return ev0.elapsed_time(ev1) / reps * 1e3

    def eager_us(fn, reps):
        for i in range(args.warmup):
            fn(i)
        torch.cuda.synchronize()
        ev0.record(stream)
        for i in range(reps):
            fn(i)
        ev1.record(stream)
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / reps * 1e3

    settled_ms, _, ceiling = settle_and_read_ceiling(ta, torch, dev, stream, args.settle_ms)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    tiny = torch.zeros(16, dtype=torch.uint8, device=dev)
    res = {"mode": "floor", "settle_ms": round(settled_ms, 1), "read_ceiling_GB_per_s": round(ceiling, 1)}
    res["empty_launch_us"] = round(graph_us(lambda i: ta.stream_read(tiny, sink), args.steps), 2)

    cw = W.COMBINE_WORKLOADS["combine_64x128"]
    ci = W.make_combine_inputs(cw, args.seed)
    nbytes = (ci.partial_o.nbytes + ci.partial_lse.nbytes) + cw.B * cw.H * (cw.d + 1) * 4
    copies = max(1, math.ceil(args.min_rotation_bytes / nbytes))
    pos = [torch.from_numpy(ci.partial_o).to(dev) for _ in range(copies)]
    pls = [torch.from_numpy(ci.partial_lse).to(dev) for _ in range(copies)]
    flat = [torch.empty(nbytes, dtype=torch.uint8, device=dev) for _ in range(copies)]
    out = torch.empty(cw.B, cw.H, cw.d, dtype=torch.float32, device=dev)
    lse = torch.empty(cw.B, cw.H, dtype=torch.float32, device=dev)
    res["combine_bytes"] = nbytes
    res["read_combine_bytes_us"] = round(graph_us(lambda i: ta.stream_read(flat[i % copies], sink), args.steps), 2)
    res["combine_us"] = round(graph_us(lambda i: ta.combine(pos[i % copies], pls[i % copies], out=out, lse=lse),
                                       args.steps), 2)
    del pos, pls, flat

    wl = W.WORKLOADS["gqa8b_128k"]
    inp = W.make_decode_inputs(wl, args.seed)
    to = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    q, k0, v0 = to(inp.q), to(inp.k), to(inp.v)
    ncopies = max(1, math.ceil(args.min_rotation_bytes / (2 * k0.numel() * 2)))
    ks, vs = [k0] + [k0.clone() for _ in range(ncopies - 1)], [v0] + [v0.clone() for _ in range(ncopies - 1)]
    P = -(-wl.N // wl.chunk)
    po = torch.empty(wl.B, wl.Hq, P, wl.d, dtype=torch.float32, device=dev)
    pl = torch.empty(wl.B, wl.Hq, P, dtype=torch.float32, device=dev)
    o1 = torch.empty(wl.B, wl.Hq, wl.d, dtype=torch.float32, device=dev)
    l1 = torch.empty(wl.B, wl.Hq, dtype=torch.float32, device=dev)
    part = lambda i: ta.partial(q, ks[i % ncopies], vs[i % ncopies], None, chunk=wl.chunk, partial_o=po, partial_lse=pl)

    def part_empty(i):
        part(i)
        ta.stream_read(tiny, sink)

    def part_combine(i):
        part(i)
        ta.combine(po, pl, out=o1, lse=l1)

    dec = lambda i: ta.decode(q, ks[i % ncopies], vs[i % ncopies], None, chunk=wl.chunk, out=o1, lse=l1)
    step = {"workload": wl.name}
    # generating the inputs left the device idle: settle again, then time the four
    # loops in turn, three times over, and keep each one's median
    settle_and_read_ceiling(ta, torch, dev, stream, args.settle_ms)
    loops = (("partial_us", part), ("partial_then_empty_launch_us", part_empty),
             ("partial_then_combine_us", part_combine), ("decode_us", dec))
    times = {name: [] for name, _ in loops}
    for _ in range(3):
        for name, f in loops:
            times[name].append(eager_us(f, args.steps))
    for name, _ in loops:
        step[name] = round(sorted(times[name])[1], 2)
    step["combine_alone_us"] = round(graph_us(lambda i: ta.combine(po, pl, out=o1, lse=l1), args.steps), 2)
    res["step_128k"] = step
    print(json.dumps(res))
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="gqa8b_128k")
    ap.add_argument("--seed", type=int, default=1)
    ap.add_argument("--chunk", type=int, default=0, help="override the workload's chunk")
    ap.add_argument("--min-rotation-bytes", type=float, default=2 * 2**30)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--settle-ms", type=float, default=100.0,
                    help="device time of streaming reads run before the warmup steps (0: none)")
    ap.add_argument("--suggested-chunk", action="store_true",
                    help="also time the step at the chunk ta_suggest_chunk returns (reported as suggested_chunk)")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle time for the CPU baseline")
    ap.add_argument("--mode", choices=["step", "partial", "copy", "combine", "floor"], default="step",
                    help="step: the benchmark line (default); partial: only the timed partial-kernel launches "
                         "(for counter runs); copy: a plain device copy of --copy-mib MiB (counter calibration); "
                         "combine: the standalone ta_combine workload (64 fp32 states per head, 32 x 32 heads); "
                         "floor: launch and streaming floors of the merge stage")
    ap.add_argument("--copy-mib", type=int, default=1024)
    ap.add_argument("--n-parts", type=int, default=0,
                    help="combine mode: states per row (default: the workload's 64)")
    ap.add_argument("--arity", type=lambda a: a if a == "chain" else int(a), default=None,
                    help="combine mode: time ta_combine_k with this branching factor (2..16), or "
                         "ta_combine_chain with 'chain', instead of ta_combine")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this single-GPU decode path has no multi-GPU mode "
              "(run with --gpus 1).", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import softmax_tree_reduction_amd as ta
    import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    wl = W.WORKLOADS[args.workload]
    chunk = args.chunk or wl.chunk
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.mode == "copy":
        # a plain copy of known size: each launch reads and writes copy-mib MiB
        n = args.copy_mib * 2**20 // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(args.warmup + args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"mode": "copy", "bytes_read_per_launch": n * 4, "bytes_written_per_launch": n * 4,
                          "launches": args.warmup + args.steps}))
        return 0
    if args.mode == "combine":
        return bench_combine(args, dev)
    if args.mode == "floor":
        return bench_floor(args, dev)
    print(f"bench: generating {wl.name} (seed {args.seed})", file=sys.stderr, flush=True)
    inp = W.make_decode_inputs(wl, args.seed)
    step_bytes = algorithmic_bytes(wl, inp.seqlens)

    def to_dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    q = to_dev(inp.q)
    # ragged batches pass their lengths; when every sequence fills the cache, none are passed
    sl = torch.from_numpy(inp.seqlens.astype(np.int32)).to(dev) if wl.ragged is not None else None
    k0, v0 = to_dev(inp.k), to_dev(inp.v)
    cache_bytes = k0.numel() * k0.element_size() * 2
    copies = max(1, math.ceil(args.min_rotation_bytes / cache_bytes))
    ks, vs = [k0], [v0]
    for _ in range(copies - 1):
        ks.append(k0.clone())
        vs.append(v0.clone())
    print(f"bench: {copies} resident copies of the {cache_bytes / 2**20:.0f} MiB cache", file=sys.stderr, flush=True)

    stream = torch.cuda.current_stream(dev)
    P = -(-wl.N // chunk)
    if args.mode == "partial":
        po = torch.empty(wl.B, wl.Hq, P, wl.d, dtype=torch.float32, device=dev)
        pl = torch.empty(wl.B, wl.Hq, P, dtype=torch.float32, device=dev)
        for i in range(args.warmup + args.steps):
            ta.partial(q, ks[i % copies], vs[i % copies], sl, chunk=chunk, partial_o=po, partial_lse=pl)
        torch.cuda.synchronize()
        print(json.dumps({"mode": "partial", "workload": wl.name, "launches": args.warmup + args.steps,
                          "algorithmic_bytes_per_launch": step_bytes - wl.B * wl.Hq * (wl.d + 1) * 4}))
        return 0

    # parity of this launch configuration on sampled rows before timing
    import oracle
    out, lse = ta.decode(q, k0, v0, sl, chunk=chunk)
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(0).choice(wl.B * wl.Hq, size=min(8, wl.B * wl.Hq), replace=False))
    ro, rl = oracle.decode(inp.q, inp.k, inp.v, inp.seqlens, rows=rows)
    o = out.cpu().numpy().reshape(-1, wl.d)[rows]
    l_ = lse.cpu().numpy().reshape(-1)[rows]
    tol = 4e-3 if wl.dtype == "bf16" else 1e-5
    perr = float(np.abs(o - ro).max())
    lerr = float((np.abs(l_ - rl) / np.maximum(1.0, np.abs(rl))).max())
    if not (perr <= tol and lerr <= 1e-4):
        print(f"bench: parity check failed (out err {perr}, lse err {lerr})", file=sys.stderr)
        return 1
    print(f"bench: parity on {len(rows)} sampled rows ok (max|out-oracle| {perr:.2e}, lse rel {lerr:.2e})",
          file=sys.stderr, flush=True)

    # ---- settle, then the practical read ceiling (before anything is timed)
    settled_ms, settle_reads, ceiling = settle_and_read_ceiling(ta, torch, dev, stream, args.settle_ms)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    print(f"bench: settled {settled_ms:.0f} ms ({settle_reads} reads of 1 GiB), read ceiling {ceiling:.0f} GB/s",
          file=sys.stderr, flush=True)

    # ---- whole step: ta_decode (partial kernel + tree merge)
    for i in range(args.warmup):
        ta.decode(q, ks[i % copies], vs[i % copies], sl, chunk=chunk, out=out, lse=lse)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        ta.decode(q, ks[i % copies], vs[i % copies], sl, chunk=chunk, out=out, lse=lse)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    ms_step = ev0.elapsed_time(ev1) / args.steps

    # the spread of the timed loop itself: the same K-step loop, timed the same way,
    # run 5 more times (the per-step mean of each run)
    loop_means = [ms_step]
    for _ in range(5):
        ev0.record(stream)
        for i in range(args.steps):
            ta.decode(q, ks[i % copies], vs[i % copies], sl, chunk=chunk, out=out, lse=lse)
        ev1.record(stream)
        torch.cuda.synchronize()
        loop_means.append(ev0.elapsed_time(ev1) / args.steps)
    loop_means.sort()

    # the spread of single steps, from a separate pass with an event after every step
    # (each event costs a few µs of its own, so these run longer than `value`'s loop)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ev0.record(stream)
    for i in range(args.steps):
        ta.decode(q, ks[i % copies], vs[i % copies], sl, chunk=chunk, out=out, lse=lse)
        marks[i].record(stream)
    torch.cuda.synchronize()
    per_step = sorted([ev0.elapsed_time(marks[0])] + [marks[i - 1].elapsed_time(marks[i]) for i in range(1, args.steps)])
    pct = lambda f: per_step[min(len(per_step) - 1, int(round(f * (len(per_step) - 1))))] * 1e3

    # the same step with warm caches: one cache copy every time (reported apart, not `value`)
    ev0.record(stream)
    for _ in range(args.steps):
        ta.decode(q, k0, v0, sl, chunk=chunk, out=out, lse=lse)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms_warm = ev0.elapsed_time(ev1) / args.steps
    print(f"bench: {args.steps} steps, {ms_step * 1e3:.1f} us/step (host wall {wall / args.steps * 1e6:.1f} us/step)",
          file=sys.stderr, flush=True)

    # ---- the same steps replayed from one captured graph through the allocation-free
    # entry point (what a caller that captures its decode loop gets; reported apart)
    graph_us = None
    try:
        side = torch.cuda.Stream(dev)
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            ta.decode_noalloc(q, ks[0], vs[0], sl, chunk=chunk, out=out, lse=lse)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(args.steps):
                ta.decode_noalloc(q, ks[i % copies], vs[i % copies], sl, chunk=chunk, out=out, lse=lse)
        graph.replay()
        torch.cuda.synchronize()
        # capturing and instantiating the graph left the device idle: settle it again
        settle_and_read_ceiling(ta, torch, dev, stream, args.settle_ms)
        reps = []
        for _ in range(3):  # the median of three timed replays
            ev0.record(stream)
            graph.replay()
            ev1.record(stream)
            torch.cuda.synchronize()
            reps.append(ev0.elapsed_time(ev1) / args.steps * 1e3)
        graph_us = round(sorted(reps)[1], 2)
        del graph
    except ta.TreeAttnError as e:  # a step larger than the static scratch
        print(f"bench: no graph replay ({e})", file=sys.stderr, flush=True)

    # ---- the same step at the chunk ta_suggest_chunk gives (reported apart, not `value`)
    # (opt-in: the default run launches the partial kernel at the workload's chunk only,
    # so a kernel trace of it averages one grid)
    alt_chunk = ta.suggest_chunk(wl.B, wl.Hq, wl.Hkv, wl.N)
    alt = None
    if args.suggested_chunk and alt_chunk != chunk:
        for i in range(args.warmup):
            ta.decode(q, ks[i % copies], vs[i % copies], sl, chunk=alt_chunk, out=out, lse=lse)
        torch.cuda.synchronize()
        ev0.record(stream)
        for i in range(args.steps):
            ta.decode(q, ks[i % copies], vs[i % copies], sl, chunk=alt_chunk, out=out, lse=lse)
        ev1.record(stream)
        torch.cuda.synchronize()
        ms_alt = ev0.elapsed_time(ev1) / args.steps
        alt = {"chunk": alt_chunk, "us_per_step": round(ms_alt * 1e3, 2),
               "GB_per_s": round(step_bytes / (ms_alt * 1e-3) / 1e9, 2),
               "note": "same workload and timing, at the chunk ta_suggest_chunk returns; not value"}

    # ---- dominant kernel alone: ta_partial over the same rotation
    po = torch.empty(wl.B, wl.Hq, P, wl.d, dtype=torch.float32, device=dev)
    pl = torch.empty(wl.B, wl.Hq, P, dtype=torch.float32, device=dev)
    for i in range(args.warmup):
        ta.partial(q, ks[i % copies], vs[i % copies], sl, chunk=chunk, partial_o=po, partial_lse=pl)
    torch.cuda.synchronize()
    ev0.record(stream)
    for i in range(args.steps):
        ta.partial(q, ks[i % copies], vs[i % copies], sl, chunk=chunk, partial_o=po, partial_lse=pl)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms_partial = ev0.elapsed_time(ev1) / args.steps

    # ---- merge alone on the partial states, replayed from a captured graph so that
    # the host's per-call cost does not hide the device time
    for _ in range(args.warmup):
        ta.combine(po, pl, out=out, lse=lse)
    torch.cuda.synchronize()
    side = torch.cuda.Stream(dev)
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        ta.combine(po, pl, out=out, lse=lse)
    stream.wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(args.steps):
            ta.combine(po, pl, out=out, lse=lse)
    graph.replay()
    torch.cuda.synchronize()
    ev0.record(stream)
    graph.replay()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms_combine = ev0.elapsed_time(ev1) / args.steps
    del graph

    partial_bytes = step_bytes - wl.B * wl.Hq * (wl.d + 1) * 4  # K, V and q; out/lse belong to the merge
    achieved = partial_bytes / (ms_partial * 1e-3) / 1e9
    traffic = measured_traffic(wl.name)
    gbs = step_bytes / (ms_step * 1e-3) / 1e9

    cpu = None
    if not args.no_cpu_baseline:
        print("bench: timing the CPU oracle", file=sys.stderr, flush=True)
        cpu = cpu_baseline(inp, wl, args.cpu_budget)

    res = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "us_per_step": round(ms_step * 1e3, 2),
        "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "us_per_step_loops": {"median": round(loop_means[len(loop_means) // 2] * 1e3, 2),
                              "min": round(loop_means[0] * 1e3, 2), "max": round(loop_means[-1] * 1e3, 2),
                              "loops": len(loop_means),
                              "note": "per-step mean of the timed K-step loop and of 5 more runs of it, timed alike"},
        "us_per_step_dist": {"median": round(pct(0.5), 2), "p10": round(pct(0.1), 2), "p90": round(pct(0.9), 2),
                             "note": "single steps from a separate pass with an event recorded after every step; "
                                     "each event adds its own few µs, so these run longer than the timed loop"},
        "us_per_step_warm": round(ms_warm * 1e3, 2),
        "us_per_step_graph_noalloc": graph_us,
        "suggested_chunk": alt,
        "read_ceiling": {"value": round(ceiling, 1), "unit": "GB/s", "kernel": "ta_stream_read",
                         "bytes_per_launch": 2**30, "step_pct_of_ceiling": round(100 * gbs / ceiling, 2)},
        "settle": {"ms": round(settled_ms, 1), "kernel": "ta_stream_read", "launches": settle_reads,
                   "note": "streaming reads before the warmup steps, so the timed steps run at the device's steady speed"},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.B, "q_heads": wl.Hq, "kv_heads": wl.Hkv, "head_dim": wl.d,
                   "context": wl.N, "chunk": chunk, "partials": P, "tree_levels": math.ceil(math.log2(P)) if P > 1 else 0,
                   "algorithmic_bytes_per_step": step_bytes, "cache_copies": copies, "seed": args.seed,
                   "generator": {"numpy": np.__version__,
                                 "sha256_first_mib": {n: hashlib.sha256(a.reshape(-1).view(np.uint8)[:2**20].tobytes())
                                                      .hexdigest()[:16] for n, a in (("q", inp.q), ("k", inp.k), ("v", inp.v))}}},
        "kernels_us": {"partial": round(ms_partial * 1e3, 2), "combine": round(ms_combine * 1e3, 2)},
        "roofline": {"kernel": "ta_partial (partial_kernel, or partial_kernel_multi when its grid takes several chunks per workgroup)", "bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "algorithmic_bytes_per_launch": partial_bytes,
                     "frac_of_read_ceiling": round(achieved / ceiling, 4)},
        "parity": {"rows": len(rows), "max_abs_out_err": perr, "max_rel_lse_err": lerr},
        "cpu_baseline": cpu,
    }
    print(json.dumps(res))
    return 0


if __name__ == "__main__":
    sys.exit(main())
