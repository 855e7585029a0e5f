"""bench.py on the host: the one-GPU contract and the bytes its headline
counts.

  * `--gpus N` with N above 1 exits with a message before touching a GPU;
  * the algorithmic K/V bytes of one layer call of the 70B-style workload
    are the pages' per-token figure for that model (327,680 bytes per token
    over its 80 layers, `tests/golden/pages_capacity.txt`) times the
    47 x 825 tokens of the snapshot, and the FP8 workload counts each
    physical token slot its block tables address once (shared prefixes
    once), at the pages' FP8 per-token figure.
"""

import os
import subprocess
import sys

import numpy as np

import bench
import oracle.allocator
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
    assert res.stdout == ""


def test_headline_bytes_follow_the_pages_per_token_figure(pages_capacity):
    per_token_all_layers = pages_capacity["gqa_bf16_bytes_per_token"]  # 80 layers of the 70B GQA model
    plan = workloads.plan(workloads.get("gqa70b-bf16-47x825"))
    assert bench.kv_bytes_per_call(plan) * 80 == 47 * 825 * per_token_all_layers
    assert bench.kv_bytes_per_call(plan) == 158_822_400


def test_shared_prefix_blocks_count_once(pages_capacity):
    """Unique bytes = the distinct physical token slots the block tables
    address (replayed through the oracle's allocator), at the pages' FP8
    per-token figure for one layer; logical bytes count every sequence's
    whole context."""
    per_token_layer = pages_capacity["gqa_fp8_bytes_per_token"] // 80
    wl = workloads.get("fp8-prefix-32xU32768")
    plan = workloads.plan(wl)
    rp = workloads.replay(plan, oracle.allocator.BlockManager(plan.num_blocks, wl.block_size, plan.free_order))
    slots = []
    for s, ctx in enumerate(np.asarray(plan.context_lens, dtype=np.int64)):
        t = np.arange(ctx)
        slots.append(rp.block_tables[s, t // wl.block_size].astype(np.int64) * wl.block_size + t % wl.block_size)
    slots = np.concatenate(slots)
    assert bench.kv_bytes_per_call(plan, unique=False) == slots.size * per_token_layer
    assert bench.kv_bytes_per_call(plan) == np.unique(slots).size * per_token_layer
    assert np.unique(slots).size < slots.size  # the groups do share their prefixes
