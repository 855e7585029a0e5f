"""Benchmark of the paged-decode hot path on one MI355X.

A step is one decode step of the 70B-style GQA model the pages size (80 layers,
8 KV heads of 128 dims, bf16): for each of 80 layers, the new tokens' K/V are
scattered into that layer's paged pool and paged decode attention runs over
it, in one launch per layer (pkv_decode_step; two_launch_step times the
separate reshape_and_cache and decode calls for the same work).  Each layer has its own pool of 2,457 blocks (the
12 GiB budget of the pages split over 80 layers), so a step streams about
12.7 GB of KV and repeats never hit in the 256 MB last-level cache.

value = KV bytes a step must read (sum over sequences of context_len x 2 x
h_kv x head_dim x 2 B, x 80 layers) / step time, in GB/s.
roofline = the step's attention kernel: the same bytes per launch / its mean
launch duration, which is the step time over 80 when the step is one launch
per layer (HIP events on the kernel's stream around the timed loop);
traffic = HBM bytes per launch from rocprofv3 counters, reported only while
the kernel source is the one they were taken on.
copy_blocks = the block copy of copy-on-write (1,024 block pairs, K and V).
swap_blocks = preemption by swap: 1,024 scattered blocks (K and V) to pinned
host memory and back in one launch each way, GB/s against PCIe 5.0 x16.
multi_query = a speculative step: 4 new query tokens per sequence (the last 4
positions of each context, causal), the same pools; GB/s counts each cached
K/V byte once.
reshape_and_cache = the separate scatter's launch time (reported, not a
target); bytes_per_layer_call = the bytes a call moves besides the used K/V
(whole blocks, queries, output, tables, new tokens), not counted in value.
roofline.measured_stream_peaks = a 2 GiB device copy's read + write rate and
a 2 GiB float32 sum's read rate (library kernels), beside the published 8 TB/s.
cpu_baseline = the float64 oracle on whole layer calls, repeated for a
bounded time on the host with its thread pools held to one thread (the
one core it uses), and briefly with the default pools for comparison.

Prints one JSON line.  Usage: python bench.py [--steps K] [--warmup W]
"""

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged decode attention: achieved KV HBM GB/s (% of peak), seqs/s at 1 GPU"
HBM_PEAK_GBS = 8000.0
DEFAULT_WORKLOAD = "gqa70b-bf16-47x825"


# Host link of an MI355X: PCIe 5.0 x16, per direction.
PCIE_PEAK_GBS = 64.0

# Lookahead tokens per sequence of the speculative step measured beside decode.
MULTI_TOKENS = 4

# HBM bytes per launch from rocprofv3 counters (FETCH_SIZE x 2 + WRITE_SIZE:
# on a 1 GiB device copy FETCH_SIZE reads half the bytes read and WRITE_SIZE
# all the bytes written), valid only for the kernel code they were taken on
# (kernel_source_sha256) and the workload / split count they ran.
MEASURED_TRAFFIC = {
    # (kernel source sha256, workload, num_splits): bytes per launch
    ("8103bae41d746a887ca72f3e4108a73f5914051d8b08feff7eb81f5cf33815b4", "gqa70b-bf16-47x825-step", 1): 161785926,
    ("8103bae41d746a887ca72f3e4108a73f5914051d8b08feff7eb81f5cf33815b4", "gqa70b-bf16-47x825", 1): 161361920,
    ("8103bae41d746a887ca72f3e4108a73f5914051d8b08feff7eb81f5cf33815b4", "gqa70b-bf16-47x825-multi4", 1): 168399872,
    ("8103bae41d746a887ca72f3e4108a73f5914051d8b08feff7eb81f5cf33815b4", "gqa70b-bf16-47x825-b32-step", 1): 161747006,
    ("8103bae41d746a887ca72f3e4108a73f5914051d8b08feff7eb81f5cf33815b4", "gqa70b-bf16-47x825-b32", 1): 161323008,
    ("8103bae41d746a887ca72f3e4108a73f5914051d8b08feff7eb81f5cf33815b4", "gqa70b-bf16-47x825-b32-multi4", 1): 168360960,
    ("8103bae41d746a887ca72f3e4108a73f5914051d8b08feff7eb81f5cf33815b4", "gqa8b-bf16-256xU4096-step", 1): 2132160432,
    ("8103bae41d746a887ca72f3e4108a73f5914051d8b08feff7eb81f5cf33815b4", "gqa8b-bf16-256xU4096", 1): 2130032641,
    ("8103bae41d746a887ca72f3e4108a73f5914051d8b08feff7eb81f5cf33815b4", "gqa8b-bf16-256xU4096-multi4", 1): 2148940803,
    ("8103bae41d746a887ca72f3e4108a73f5914051d8b08feff7eb81f5cf33815b4", "mha-f16-64x4096-step", 1): 4299399281,
    ("8103bae41d746a887ca72f3e4108a73f5914051d8b08feff7eb81f5cf33815b4", "mha-f16-64x4096", 1): 4297254912,
    ("8103bae41d746a887ca72f3e4108a73f5914051d8b08feff7eb81f5cf33815b4", "mha-f16-64x4096-multi4", 1): 4301980672,
    ("8103bae41d746a887ca72f3e4108a73f5914051d8b08feff7eb81f5cf33815b4", "fp8-prefix-32xU32768-step", 2): 1267052557,
    ("8103bae41d746a887ca72f3e4108a73f5914051d8b08feff7eb81f5cf33815b4", "fp8-prefix-32xU32768", 2): 1267417925,
    ("8103bae41d746a887ca72f3e4108a73f5914051d8b08feff7eb81f5cf33815b4", "fp8-prefix-32xU32768-multi4", 2): 1290396874,
}


def kernel_source_sha256():
    """SHA-256 of the attention kernels' code: paged_decode.hip with its //
    comments, blank lines and runs of white space removed, so that editing a
    comment does not invalidate counters taken on the same code."""
    import hashlib
    import re
    path = os.path.join(ROOT, "paged_kv_cache_431_amd", "csrc", "paged_decode.hip")
    lines = []
    with open(path) as f:
        for line in f:
            line = re.sub(r"//.*$", "", line).strip()
            if line:
                lines.append(re.sub(r"\s+", " ", line))
    return hashlib.sha256("\n".join(lines).encode()).hexdigest()


def measured_traffic(workload, num_splits):
    """Counter-measured HBM bytes per launch, or None if the decode kernel
    changed since they were taken (or they were never taken for this case)."""
    return MEASURED_TRAFFIC.get((kernel_source_sha256(), workload, int(num_splits)))


def kv_bytes_per_call(plan, unique=True):
    """Algorithmic K+V bytes one decode call reads: used tokens only."""
    import workloads
    wl = plan.workload
    per_token = 2 * wl.h_kv * wl.head_dim * workloads.ELEMENT_BYTES[wl.kv_dtype]
    total = int(plan.context_lens.astype("int64").sum()) * per_token
    if unique and wl.layout == "shared_prefix":
        groups = -(-wl.num_seqs // wl.group_size)
        total -= (wl.num_seqs - groups) * wl.prefix_tokens * per_token
    return total


def side_bytes_per_call(plan, fused):
    """Bytes a layer call moves besides the used K/V tokens, reported beside
    the headline figure but not counted in it: the whole blocks the used
    tokens lie in (the tail slots of each last block are fetched with it),
    the per-sequence bytes the shared prefix blocks would take if every
    sequence had its own copy, the queries, the output, the block tables and
    context lengths, and the new tokens' K/V."""
    import workloads
    wl = plan.workload
    e_kv = workloads.ELEMENT_BYTES[wl.kv_dtype]
    per_token = 2 * wl.h_kv * wl.head_dim * e_kv
    ctx = plan.context_lens.astype("int64")
    blocks = -(-ctx // wl.block_size)
    allocated = int(blocks.sum()) * wl.block_size * per_token
    if wl.layout == "shared_prefix":
        groups = -(-wl.num_seqs // wl.group_size)
        allocated -= (wl.num_seqs - groups) * wl.prefix_tokens * per_token
    new_tok = wl.num_seqs * 2 * wl.h_kv * wl.head_dim
    return {
        "kv_used_bytes": kv_bytes_per_call(plan),
        "kv_logical_bytes": kv_bytes_per_call(plan, unique=False),
        "kv_allocated_bytes": allocated,
        "q_bytes": wl.num_seqs * wl.h_q * wl.head_dim * workloads.ELEMENT_BYTES[wl.q_dtype],
        "out_bytes": wl.num_seqs * wl.h_q * wl.head_dim * 4,
        "block_table_bytes": int(sum(int(b) for b in blocks)) * 4,
        "context_len_bytes": wl.num_seqs * 4,
        "new_kv_read_bytes": new_tok * workloads.ELEMENT_BYTES[wl.new_dtype] if fused else 0,
        "new_kv_written_bytes": new_tok * e_kv if fused else 0,
    }


def stream_peaks(dev, nbytes, reps=10):
    """Streaming rates the memory system gives plain library kernels on
    nbytes: a device-to-device copy (the runtime's copy kernel; read + write
    bytes) and a float32 sum (torch's reduction; bytes read), GB/s."""
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)

    def median_ms(fn):
        for _ in range(3):
            fn()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a, b in evs:
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        return sorted(a.elapsed_time(b) for a, b in evs)[reps // 2]

    copy_ms = median_ms(lambda: dst.copy_(src))
    sum_ms = median_ms(lambda: torch.sum(src))
    del src, dst
    torch.cuda.empty_cache()
    return 2 * nbytes / (copy_ms * 1e-3) / 1e9, nbytes / (sum_ms * 1e-3) / 1e9


def cpu_baseline(plan, rp, tensors, budget_s, blas_budget_s):
    """Time the oracle on whole layer calls of the workload (the scatter of the
    new tokens, then float64 attention one sequence at a time), repeating the
    layer until about budget_s seconds of host work are done, with every
    thread pool held to one thread: the oracle walks one sequence and head at
    a time through small float64 products, so one core is what it uses.  A
    second run of blas_budget_s seconds leaves the BLAS and torch thread pools
    at their defaults and reports their size beside the rate, which shows
    that more threads do not speed it up."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_info, threadpool_limits

    import oracle.attention
    import oracle.scatter

    wl = plan.workload
    bits = {torch.float32: (torch.int32, np.uint32), torch.float16: (torch.int16, np.uint16),
            torch.bfloat16: (torch.int16, np.uint16), torch.uint8: (torch.uint8, np.uint8)}
    to_np = lambda x: x.view(bits[x.dtype][0]).cpu().numpy().view(bits[x.dtype][1])
    q, kc, vc = to_np(tensors.q), to_np(tensors.k_cache), to_np(tensors.v_cache)
    nk, nv = to_np(tensors.new_k), to_np(tensors.new_v)
    per_call = kv_bytes_per_call(plan)

    def run(budget):
        done_calls = 0
        t0 = time.perf_counter()
        while True:
            kc2, vc2 = oracle.scatter.reshape_and_cache(nk, nv, kc, vc, rp.slot_mapping, in_dtype=wl.new_dtype,
                                                        kv_dtype=wl.kv_dtype, block_size=wl.block_size,
                                                        k_scale=tensors.k_scale, v_scale=tensors.v_scale)
            for s in range(wl.num_seqs):
                oracle.attention.paged_attention_decode(q, kc2, vc2, rp.block_tables, plan.context_lens,
                                                        q_dtype=wl.q_dtype, kv_dtype=wl.kv_dtype,
                                                        block_size=wl.block_size,
                                                        scale=1.0 / math.sqrt(wl.head_dim),
                                                        k_scale=tensors.k_scale, v_scale=tensors.v_scale, seqs=[s])
            done_calls += 1
            if time.perf_counter() - t0 > budget:
                return done_calls, time.perf_counter() - t0

    def pool_threads():
        return int(max([i.get("num_threads", 1) for i in threadpool_info()] or [1]))

    def sample(calls, dt):
        return (f"{calls} repeats of one layer call of {wl.name} ({wl.num_seqs} sequences: scatter of the new "
                f"tokens, then float64 attention one sequence at a time), {dt:.1f} s")

    torch_threads = torch.get_num_threads()
    with threadpool_limits(limits=1):
        torch.set_num_threads(1)
        try:
            calls, dt = run(budget_s)
            assert pool_threads() == 1
        finally:
            torch.set_num_threads(torch_threads)
    result = {"value": round(calls * per_call / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
              "seqs_per_s": round(calls * wl.num_seqs / dt, 3), "host_cpus": os.cpu_count(),
              "sample": sample(calls, dt) + ", every thread pool held to one thread"}
    if blas_budget_s > 0:
        calls2, dt2 = run(blas_budget_s)
        result["default_thread_pools"] = {
            "value": round(calls2 * per_call / dt2 / 1e9, 4), "unit": "GB/s", "blas_threads": pool_threads(),
            "torch_threads": torch_threads, "sample": sample(calls2, dt2),
            "note": "the same oracle with the BLAS and torch pools at their default sizes; its products are too "
                    "small to spread over them, so it still runs on about one core"}
    return result


def swap_measurement(pkv, t, plan, wl, stream, n_pairs, _hbm_peak):
    """Preemption by swap: n_pairs scattered blocks (K and V) of one layer pool
    to a pinned host pool and back, one launch each way; the latency of a
    one-block swap; and, for reference, the DMA engines' rate for one
    contiguous pinned buffer of the same size."""
    import numpy as np
    import torch
    block_bytes = wl.h_kv * wl.block_size * wl.head_dim * t.k_cache.element_size()
    shape = (n_pairs,) + tuple(t.k_cache.shape[1:])
    hk = torch.empty(shape, dtype=t.k_cache.dtype, pin_memory=True)
    hv = torch.empty(shape, dtype=t.v_cache.dtype, pin_memory=True)
    dev_blocks = np.random.default_rng(11).permutation(plan.num_blocks)[:n_pairs]
    out_pairs = torch.from_numpy(np.stack([dev_blocks, np.arange(n_pairs)], axis=1).astype(np.int32)).cuda()
    in_pairs = torch.from_numpy(np.stack([np.arange(n_pairs), dev_blocks], axis=1).astype(np.int32)).cuda()

    def timed(fn, reps):
        for _ in range(3):
            fn()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a, b in evs:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        return sorted(a.elapsed_time(b) for a, b in evs)[reps // 2]  # median, ms

    moved = n_pairs * 2 * block_bytes
    d2h = timed(lambda: pkv.pkv_swap_blocks(hk, hv, t.k_cache, t.v_cache, out_pairs, stream=stream), 10)
    h2d = timed(lambda: pkv.pkv_swap_blocks(t.k_cache, t.v_cache, hk, hv, in_pairs, stream=stream), 10)
    one_d2h = timed(lambda: pkv.pkv_swap_blocks(hk, hv, t.k_cache, t.v_cache, out_pairs[:1], stream=stream), 20)
    one_h2d = timed(lambda: pkv.pkv_swap_blocks(t.k_cache, t.v_cache, hk, hv, in_pairs[:1], stream=stream), 20)
    flat_h = torch.empty(moved, dtype=torch.uint8, pin_memory=True)
    flat_d = torch.empty(moved, dtype=torch.uint8, device="cuda")
    dma_d2h = timed(lambda: flat_h.copy_(flat_d, non_blocking=True), 10)
    dma_h2d = timed(lambda: flat_d.copy_(flat_h, non_blocking=True), 10)
    gbps = lambda ms: round(moved / (ms * 1e-3) / 1e9, 2)
    return {"pairs": n_pairs, "bytes_per_call": moved, "peak_GBps": PCIE_PEAK_GBS,
            "d2h_us": round(d2h * 1e3, 2), "d2h_GBps": gbps(d2h), "d2h_frac": round(gbps(d2h) / PCIE_PEAK_GBS, 4),
            "h2d_us": round(h2d * 1e3, 2), "h2d_GBps": gbps(h2d), "h2d_frac": round(gbps(h2d) / PCIE_PEAK_GBS, 4),
            "one_block_d2h_us": round(one_d2h * 1e3, 2), "one_block_h2d_us": round(one_h2d * 1e3, 2),
            "dma_contiguous_d2h_GBps": gbps(dma_d2h), "dma_contiguous_h2d_GBps": gbps(dma_h2d)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--layers", type=int, default=80)
    ap.add_argument("--block-size", type=int, default=0, help="tokens per block (0: the workload's own, 16)")
    ap.add_argument("--splits", type=int, default=0, help="force the decode split count (0 = library's choice)")
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="seconds of oracle work for cpu_baseline (thread pools held to one thread)")
    ap.add_argument("--cpu-budget-default-threads", type=float, default=5.0,
                    help="seconds of oracle work with the default thread pools (0 skips that run)")
    ap.add_argument("--copy-peak-mib", type=int, default=2048,
                    help="buffer size of the copy and sum that measure streaming rates (0 skips them)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--settle-ms", type=float, default=50.0,
                    help="before each timed group, launch its calls back to back for this long (GPU clocks settle)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only copy a buffer of this many MiB a few times (calibrates byte counters), then exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import paged_kv_cache_431_amd as pkv
    import workloads

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = "cuda:0"
    if args.copy_probe_mib:
        # A plain device copy of known size: its FETCH_SIZE / WRITE_SIZE
        # readings per dispatch give the scale of those counters.
        n = args.copy_probe_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "copies": 4}), flush=True)
        return
    wl = workloads.get(args.workload)
    if args.block_size and args.block_size != wl.block_size:
        # same byte budget per layer pool, blocks of another size
        blocks = wl.num_blocks * wl.block_size // args.block_size if wl.num_blocks else 0
        wl = workloads.replace(wl, name=f"{wl.name}-b{args.block_size}", block_size=args.block_size,
                               num_blocks=blocks)
    plan = workloads.plan(wl)
    bm = pkv.BlockManager(plan.num_blocks, wl.block_size, plan.free_order)
    rp = workloads.replay(plan, bm)
    L = args.layers
    pools = [workloads.make_tensors(plan, rp, device=dev, poison=False, pool_seed_offset=l) for l in range(L)]
    tables = torch.from_numpy(rp.block_tables).to(dev)
    lens = torch.from_numpy(plan.context_lens).to(dev)
    slots = torch.from_numpy(rp.slot_mapping).to(dev)
    out = torch.empty(wl.num_seqs, wl.h_q, wl.head_dim, dtype=torch.float32, device=dev)
    ws = pkv.make_workspace(wl.num_seqs, wl.h_q, wl.h_kv, wl.head_dim, wl.block_size, plan.max_context_len,
                            args.splits, device=dev)
    n_splits = pkv.pkv_decode_num_splits(wl.num_seqs, wl.h_q, wl.h_kv, wl.head_dim, wl.block_size,
                                         plan.max_context_len, args.splits)
    stream = torch.cuda.current_stream()

    # Validate and marshal every launch once; the timed loop only issues them.
    decodes = [pkv.prepare_paged_attention_decode(out, t.q, t.k_cache, t.v_cache, tables, lens,
                                                  max_context_len=plan.max_context_len, k_scale=t.k_scale,
                                                  v_scale=t.v_scale, num_splits=args.splits, workspace=ws,
                                                  stream=stream) for t in pools]
    scatters = [pkv.prepare_reshape_and_cache(t.new_k, t.new_v, t.k_cache, t.v_cache, slots, k_scale=t.k_scale,
                                              v_scale=t.v_scale, stream=stream) for t in pools]
    two_launch_calls = [c for pair in zip(scatters, decodes) for c in pair]
    # One launch per layer where the library fuses the scatter into decode
    # (matrix-core configurations), the two calls otherwise: the same bits.
    fused = True
    try:
        steps_fused = [pkv.prepare_decode_step(out, t.q, t.new_k, t.new_v, t.k_cache, t.v_cache, tables, lens,
                                               max_context_len=plan.max_context_len, workspace=ws, k_scale=t.k_scale,
                                               v_scale=t.v_scale, num_splits=args.splits, stream=stream)
                       for t in pools]
        steps_fused[0]()
    except pkv.PkvError as e:
        if e.status != pkv.PKV_EUNSUPPORTED:
            raise
        fused, steps_fused = False, []
    layer_calls = steps_fused if fused else two_launch_calls
    kernel_calls = steps_fused if fused else decodes

    def settle(calls):
        # The GPU's clocks take a few milliseconds of load to settle after an
        # idle gap (launch durations rise and fall again by up to 15 % over
        # them in a kernel trace), so each timed group starts after its own
        # calls have run back to back for settle_ms.  This is untimed.
        t0 = time.perf_counter()
        while True:
            for call in calls:
                call()
            torch.cuda.synchronize()
            if (time.perf_counter() - t0) * 1e3 >= args.settle_ms:
                return

    def time_step(calls):
        settle(calls)
        for _ in range(args.warmup):
            for call in calls:
                call()
        torch.cuda.synchronize()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record(stream)
        for _ in range(args.steps):
            for call in calls:
                call()
        end.record(stream)
        torch.cuda.synchronize()
        return start.elapsed_time(end) / args.steps

    ms_step = time_step(layer_calls)
    ms_two = time_step(two_launch_calls) if fused else ms_step

    # The step's attention kernel: where the step is one launch per layer
    # (the decode step kernel), the timed step loop above is nothing but L
    # back-to-back launches of it, so its mean launch duration is the step
    # time over L (by construction never more than the step).  Otherwise the
    # decode kernel alone is timed the same way in a loop of its own.  An
    # event pair around each single launch is also kept (it adds the event
    # and dispatch overhead).
    reps = max(1, min(5, args.steps))
    if fused:
        mean_launch_ms = ms_step / L
    else:
        settle(kernel_calls)
        batch = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a, b in batch:
            a.record(stream)
            for call in kernel_calls:
                call()
            b.record(stream)
        torch.cuda.synchronize()
        mean_launch_ms = sum(a.elapsed_time(b) for a, b in batch) / (reps * L)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps * L)]
    for r in range(reps):
        for l, call in enumerate(kernel_calls):
            a, b = evs[r * L + l]
            a.record(stream)
            call()
            b.record(stream)
    torch.cuda.synchronize()
    launch_ms = sorted(a.elapsed_time(b) for a, b in evs)
    decode_only_ms = mean_launch_ms
    if fused:  # the plain decode kernel over the same pools, for comparison
        settle(decodes)
        batch = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a, b in batch:
            a.record(stream)
            for call in decodes:
                call()
            b.record(stream)
        torch.cuda.synchronize()
        decode_only_ms = sum(a.elapsed_time(b) for a, b in batch) / (reps * L)
    # reshape_and_cache alone over the same pools (launch-bound: reported, not a target)
    batch = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in batch:
        a.record(stream)
        for call in scatters:
            call()
        b.record(stream)
    torch.cuda.synchronize()
    scatter_ms = sum(a.elapsed_time(b) for a, b in batch) / (reps * L)
    sevs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(L)]
    for (a, b), call in zip(sevs, scatters):
        a.record(stream)
        call()
        b.record(stream)
    torch.cuda.synchronize()
    scatter_iso = sorted(a.elapsed_time(b) for a, b in sevs)
    pct = lambda xs, f: xs[min(len(xs) - 1, int(f * len(xs)))]

    per_call = kv_bytes_per_call(plan)
    step_bytes = per_call * L
    value = step_bytes / (ms_step * 1e-3) / 1e9
    achieved = per_call / (mean_launch_ms * 1e-3) / 1e9
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_ms": args.settle_ms,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.kv_dtype,
        "data": "synthetic (seeded N(0,1) K/V/q; block tables from the block manager over a shuffled free list)",
        "config": {"workload": wl.name, "layers": L, "num_seqs": wl.num_seqs,
                   "context_lens": "825 each" if len(set(plan.context_lens.tolist())) == 1 else "mixed",
                   "max_context_len": plan.max_context_len, "h_q": wl.h_q, "h_kv": wl.h_kv,
                   "head_dim": wl.head_dim, "block_size": wl.block_size, "kv_dtype": wl.kv_dtype,
                   "q_dtype": wl.q_dtype, "pool_blocks_per_layer": plan.num_blocks, "num_splits": n_splits,
                   "kv_bytes_per_layer_call": per_call, "kv_bytes_per_step": step_bytes},
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "launches_per_layer": 1 if fused else 2,
        "two_launch_step": {"ms_per_step": round(ms_two, 4), "value": round(step_bytes / (ms_two * 1e-3) / 1e9, 2),
                            "note": "pkv_reshape_and_cache then pkv_paged_attention_decode per layer"},
        "seqs_per_s": round(wl.num_seqs / (ms_step * 1e-3 / L), 1),
        "decode_steps_per_s": round(1000.0 / ms_step, 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(wl.name + ("-step" if fused else ""), n_splits),
                     "kernel": ("decode_mfma_kernel (decode step, new tokens written in-kernel)" if fused else
                                "decode_mfma_kernel" if wl.kv_dtype != "f32" else "decode_vector_kernel"),
                     "mean_launch_us": round(mean_launch_ms * 1e3, 3),
                     "mean_launch_source": ("the timed step loop (ms_per_step / layers)" if fused else
                                            "back-to-back decode launches over the layer pools"),
                     "isolated_launch_median_us": round(launch_ms[len(launch_ms) // 2] * 1e3, 3),
                     "isolated_launch_p10_us": round(pct(launch_ms, 0.1) * 1e3, 3),
                     "isolated_launch_p90_us": round(pct(launch_ms, 0.9) * 1e3, 3),
                     "isolated_launches": len(launch_ms),
                     "measured_stream_peaks": None,  # filled in last (below)
                     "algorithmic_bytes_per_launch": per_call,
                     "kernel_source_sha256": kernel_source_sha256(),
                     "decode_only_mean_launch_us": round(decode_only_ms * 1e3, 3)},
    }
    # copy-on-write block copy: disjoint (src, dst) block pairs of one layer pool
    n_pairs = min(1024, plan.num_blocks // 2)
    perm = np.random.default_rng(7).permutation(plan.num_blocks)
    pairs = torch.from_numpy(np.stack([perm[:n_pairs], perm[n_pairs:2 * n_pairs]], axis=1).astype(np.int32)).to(dev)
    t0 = pools[0]
    for _ in range(3):
        pkv.pkv_copy_blocks(t0.k_cache, t0.v_cache, pairs, stream=stream)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(10):
        pkv.pkv_copy_blocks(t0.k_cache, t0.v_cache, pairs, stream=stream)
    b.record(stream)
    torch.cuda.synchronize()
    copy_ms = a.elapsed_time(b) / 10
    block_bytes = wl.h_kv * wl.block_size * wl.head_dim * workloads.ELEMENT_BYTES[wl.kv_dtype]
    moved = n_pairs * 2 * block_bytes * 2  # K and V blocks, each read once and written once
    result["bytes_per_layer_call"] = side_bytes_per_call(plan, fused)
    result["reshape_and_cache"] = {"mean_launch_us": round(scatter_ms * 1e3, 3),
                                   "isolated_launch_median_us": round(scatter_iso[len(scatter_iso) // 2] * 1e3, 3),
                                   "new_tokens": wl.num_seqs,
                                   "note": "the two-launch path's scatter alone; the decode step writes the new "
                                           "tokens inside its attention kernel"}
    result["copy_blocks"] = {"pairs": n_pairs, "block_bytes_per_pool": block_bytes, "us_per_call": round(copy_ms * 1e3, 3),
                             "read_plus_write_GBps": round(moved / (copy_ms * 1e-3) / 1e9, 1),
                             "frac_of_hbm_peak": round(moved / (copy_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    # several new query tokens per sequence: a speculative step that verifies
    # MULTI_TOKENS lookahead tokens, the last MULTI_TOKENS positions of each
    # context, over the same layer pools and tables (causal within them)
    m = MULTI_TOKENS
    qm, qs = workloads.multi_queries(wl, [m] * wl.num_seqs, device=dev)
    qs_t = torch.from_numpy(qs).to(dev)
    out_m = torch.empty(qm.shape[0], wl.h_q, wl.head_dim, dtype=torch.float32, device=dev)
    ws_m = pkv.make_multi_workspace(wl.num_seqs, wl.h_q, wl.h_kv, wl.head_dim, wl.block_size, m,
                                    plan.max_context_len, 0, device=dev)
    multis = [pkv.prepare_paged_attention_multi(out_m, qm, t.k_cache, t.v_cache, tables, lens, qs_t, max_query_len=m,
                                                max_context_len=plan.max_context_len, workspace=ws_m,
                                                k_scale=t.k_scale, v_scale=t.v_scale, stream=stream) for t in pools]
    settle(multis)
    batch = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in batch:
        a.record(stream)
        for call in multis:
            call()
        b.record(stream)
    torch.cuda.synchronize()
    multi_ms = sum(a.elapsed_time(b) for a, b in batch) / (reps * L)
    result["multi_query"] = {
        "new_tokens_per_seq": m, "query_rows": int(qm.shape[0]),
        "num_splits": pkv.pkv_multi_num_splits(wl.num_seqs, wl.h_q, wl.h_kv, wl.head_dim, wl.block_size, m,
                                               plan.max_context_len, 0),
        "mean_launch_us": round(multi_ms * 1e3, 3),
        "traffic": measured_traffic(f"{wl.name}-multi{m}", pkv.pkv_multi_num_splits(
            wl.num_seqs, wl.h_q, wl.h_kv, wl.head_dim, wl.block_size, m, plan.max_context_len, 0)),
        "kv_GBps": round(per_call / (multi_ms * 1e-3) / 1e9, 2),
        "frac_of_hbm_peak": round(per_call / (multi_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    result["swap_blocks"] = swap_measurement(pkv, pools[0], plan, wl, stream, n_pairs, HBM_PEAK_GBS)
    # The plain-kernel stream rates come after every timing of the library's
    # kernels: a 2 GiB copy and sum leave the GPU measurably slower for a
    # while (a kernel timed right after them ran 5 % slower).
    if args.copy_peak_mib:
        peaks = stream_peaks(dev, args.copy_peak_mib << 20)
        result["roofline"]["measured_stream_peaks"] = {
            "copy_GBps": round(peaks[0], 1), "sum_GBps": round(peaks[1], 1),
            "buffer_bytes": args.copy_peak_mib << 20,
            "note": "device-to-device copy (read + write bytes) and float32 sum (bytes read) of one buffer, "
                    "median of 10",
            "achieved_over_sum": round(achieved / peaks[1], 4)}
    if not args.no_cpu_baseline:
        del pools, decodes, scatters, layer_calls, multis, steps_fused, two_launch_calls, kernel_calls
        torch.cuda.empty_cache()
        fresh = workloads.make_tensors(plan, rp, device=dev, poison=False, pool_seed_offset=0)  # untouched by HIP
        result["cpu_baseline"] = cpu_baseline(plan, rp, fresh, args.cpu_budget, args.cpu_budget_default_threads)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
