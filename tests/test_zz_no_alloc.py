"""pkv_paged_attention_decode_noalloc (the library's own workspace, nothing
allocated) against pkv_paged_attention_decode (a caller workspace) through
the C ABI: the same output bits on consecutive calls of different sizes
(smaller after larger and larger after smaller, with partial states of the
split over blocks in the shared array), and the oracle's rows within the
decode tolerances."""

import numpy as np
import pytest
import torch

import paged_kv_cache_431_amd as pkv
import workloads
from pkv_cases import Case, assert_close

pytestmark = pytest.mark.gpu


def _workload(name, h_q, h_kv, kv, contexts, seed):
    q = "bf16" if kv != "f32" else "f32"
    return workloads.Workload(name, len(contexts), h_q, h_kv, 128, 16, q, kv, q, seed, contexts=tuple(contexts),
                              extra_blocks=3)


def _both(c):
    """(caller-workspace output, no-alloc output) of one decode call."""
    wl = c.wl
    ref = c.decode()
    out = torch.full((wl.num_seqs, wl.h_q, wl.head_dim), float("nan"), dtype=torch.float32, device="cuda")
    pkv.pkv_paged_attention_decode_noalloc(out, c.t.q, c.t.k_cache, c.t.v_cache, c.block_tables, c.context_lens,
                                           max_context_len=c.plan.max_context_len, k_scale=c.t.k_scale,
                                           v_scale=c.t.v_scale)
    torch.cuda.synchronize()
    return ref, out


def test_noalloc_matches_the_workspace_call_on_consecutive_calls():
    rng = np.random.default_rng(91)
    long_ctx = tuple(int(x) for x in rng.integers(2000, 12000, size=10))
    cases = [
        # few pairs with long contexts: split over blocks (balanced ranges),
        # partial states in the shared array
        _workload("na-long-bf16", 16, 2, "bf16", long_ctx, 92),
        # a smaller call right after it
        _workload("na-small-bf16", 8, 2, "bf16", (1, 17, 300, 0, 900), 93),
        # more (sequence, KV head) pairs than any call before: counters beyond
        # the earlier calls' partial states
        workloads.get("gqa70b-bf16-47x825"),
        # FP8 pools, then the first call again
        _workload("na-fp8", 32, 4, "fp8", (5, 4000, 33, 16, 9000, 1), 94),
        _workload("na-long-bf16", 16, 2, "bf16", long_ctx, 92),
        # the vector path (fp32 caches)
        _workload("na-f32", 8, 2, "f32", (3, 200, 64, 0, 17), 95),
    ]
    for wl in cases:
        print(f"[case] no-alloc {wl.name} S={wl.num_seqs} h_kv={wl.h_kv} "
              f"splits={pkv.pkv_decode_num_splits(wl.num_seqs, wl.h_q, wl.h_kv, wl.head_dim, wl.block_size, max(wl.contexts))}",
              flush=True)
        c = Case(wl)
        c.scatter()
        ref, out = _both(c)
        assert torch.equal(out, ref), f"{wl.name}: no-alloc output differs from the workspace call"
        if wl.num_seqs <= 10:
            assert_close(out, c.oracle_decode(), wl.kv_dtype, label=f"no-alloc {wl.name}")


def test_noalloc_rejects_calls_beyond_its_workspace():
    """More pairs than the counters hold: refused before any launch."""
    wl = _workload("na-huge", 8, 8, "bf16", (1,), 96)
    c = Case(wl)
    q = torch.zeros((70000, 8, 128), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((70000, 8, 128), dtype=torch.float32, device="cuda")
    bt = torch.zeros((70000, 1), dtype=torch.int32, device="cuda")
    lens = torch.ones(70000, dtype=torch.int32, device="cuda")
    with pytest.raises(pkv.PkvError, match="PKV_EWORKSPACE"):
        pkv.pkv_paged_attention_decode_noalloc(out, q, c.t.k_cache, c.t.v_cache, bt, lens, max_context_len=1)
