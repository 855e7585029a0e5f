"""Pacing of the workgroups that have a compute unit to themselves.  A
one-token launch over a 16-bit cache with head_dim 128 and one workgroup per
(sequence, KV head) puts two workgroups on some CUs and one on the others
when it has between 257 and 384 of them; the lone ones with at least 32
tiles wait after each tile, which changes when they read and nothing they
compute.  The cases are 40 sequences x 8 KV heads (320 workgroups, the
70B-style layer's head shape) with ragged contexts: pairs too short to be
paced beside paced ones, empty sequences, and lengths that leave the four
waves of a workgroup unequal tile counts.  Decode, the one-launch step and
several new query tokens (up to 4 tokens of 8 query heads: two row tiles,
held by one workgroup) are paced, and so is a grid that forced splits bring
into the window (20 sequences x 8 KV heads x 2 splits), whose partial states
are merged across workgroups.  Checks:
  * every output row against the oracle;
  * the output bit-equal to the same sequences run in a grid below the
    window (the first 30 sequences: 240 workgroups, none paced);
  * the one-launch step bit-equal to scatter + decode, pools included."""

import numpy as np
import pytest
import torch

import paged_kv_cache_431_amd as pkv
import workloads
from pkv_cases import Case, assert_close

pytestmark = pytest.mark.gpu

H_Q, H_KV, D, BS = 64, 8, 128, 16
NUM_SEQS, SUBSET = 40, 30
TYPES = [("bf16", "bf16", "bf16"), ("f16", "f16", "f16")]


def contexts(seed):
    rng = np.random.default_rng(seed)
    ctx = [int(c) for c in rng.integers(512, 2001, size=NUM_SEQS)]
    short = (0, 1, 17, 300, 511)  # fewer than 32 tiles: not paced
    for i in range(0, NUM_SEQS, 5):
        ctx[i] = short[(i // 5) % len(short)]
    ctx[3], ctx[7], ctx[11] = 512, 513, 2000  # exactly 32 tiles, one past, the longest
    return tuple(ctx)


def paced_case(types, seed):
    q, kv, new = types
    name = f"paced-{q}-{kv}-hq{H_Q}-hkv{H_KV}-b{BS}-s{NUM_SEQS}"
    return workloads.Workload(name, NUM_SEQS, H_Q, H_KV, D, BS, q, kv, new, seed, contexts=contexts(seed),
                              extra_blocks=9)


def test_grid_is_inside_the_paced_window():
    """The library's own split choice keeps one workgroup per pair here, so
    the launches below are the paced ones (320 workgroups)."""
    wl = paced_case(TYPES[0], 91)
    max_ctx = workloads.plan(wl).max_context_len
    assert pkv.pkv_decode_num_splits(NUM_SEQS, H_Q, H_KV, D, BS, max_ctx, 0) == 1
    assert pkv.pkv_multi_num_splits(NUM_SEQS, H_Q, H_KV, D, BS, 4, max_ctx, 0) == 1
    assert 256 < NUM_SEQS * H_KV <= 384 and SUBSET * H_KV <= 256


@pytest.mark.parametrize("types", TYPES, ids=lambda t: "-".join(t))
def test_paced_decode(types):
    wl = paced_case(types, 91)
    print(f"[case] {wl.name} decode", flush=True)
    c = Case(wl)
    c.scatter()
    out = c.decode()
    torch.cuda.synchronize()
    assert_close(out, c.oracle_decode(), wl.kv_dtype, label=f"{wl.name} all rows")

    print(f"[case] {wl.name} unpaced subset", flush=True)
    sub = torch.empty((SUBSET, H_Q, D), dtype=torch.float32, device="cuda")
    pkv.pkv_paged_attention_decode(sub, c.t.q[:SUBSET].contiguous(), c.t.k_cache, c.t.v_cache,
                                   c.block_tables[:SUBSET].contiguous(), c.context_lens[:SUBSET].contiguous(),
                                   max_context_len=c.plan.max_context_len, k_scale=c.t.k_scale,
                                   v_scale=c.t.v_scale, num_splits=1)
    torch.cuda.synchronize()
    assert torch.equal(sub, out[:SUBSET]), f"{wl.name}: paced rows differ from the unpaced launch"


@pytest.mark.parametrize("types", TYPES, ids=lambda t: "-".join(t))
def test_paced_step(types):
    wl = paced_case(types, 93)
    print(f"[case] {wl.name} step", flush=True)
    two = Case(wl)
    two.scatter()
    ref_out = two.decode()
    torch.cuda.synchronize()
    one = Case(wl)
    out = torch.empty((wl.num_seqs, wl.h_q, wl.head_dim), dtype=torch.float32, device="cuda")
    pkv.pkv_decode_step(out, one.t.q, one.t.new_k, one.t.new_v, one.t.k_cache, one.t.v_cache, one.block_tables,
                        one.context_lens, max_context_len=one.plan.max_context_len, k_scale=one.t.k_scale,
                        v_scale=one.t.v_scale)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out), f"{wl.name}: step output differs from scatter + decode"
    assert torch.equal(one.t.k_cache.view(torch.uint8), two.t.k_cache.view(torch.uint8)), f"{wl.name}: K pool"
    assert torch.equal(one.t.v_cache.view(torch.uint8), two.t.v_cache.view(torch.uint8)), f"{wl.name}: V pool"
    assert_close(out, one.oracle_decode(), wl.kv_dtype, label=f"{wl.name} step all rows")


@pytest.mark.parametrize("types", TYPES, ids=lambda t: "-".join(t))
def test_paced_several_query_tokens(types):
    wl = paced_case(types, 95)
    ms = [(4, 3, 4, 1, 2)[i % 5] for i in range(NUM_SEQS)]  # ragged; more tokens than cached ones included
    print(f"[case] {wl.name} new tokens", flush=True)
    c = Case(wl)
    c.scatter()
    q, qs = workloads.multi_queries(wl, ms, device="cuda")
    out = c.multi(q, qs, max(ms))
    torch.cuda.synchronize()
    assert_close(out, c.oracle_multi(q, qs), wl.kv_dtype, label=f"{wl.name} several tokens")

    print(f"[case] {wl.name} new tokens, unpaced subset", flush=True)
    rows = int(qs[SUBSET])
    sub = torch.empty((rows, H_Q, D), dtype=torch.float32, device="cuda")
    pkv.pkv_paged_attention_multi(sub, q[:rows].contiguous(), c.t.k_cache, c.t.v_cache,
                                  c.block_tables[:SUBSET].contiguous(), c.context_lens[:SUBSET].contiguous(),
                                  torch.from_numpy(np.ascontiguousarray(qs[:SUBSET + 1])).cuda(),
                                  max_query_len=max(ms), max_context_len=c.plan.max_context_len,
                                  k_scale=c.t.k_scale, v_scale=c.t.v_scale, num_splits=1)
    torch.cuda.synchronize()
    assert torch.equal(sub, out[:rows]), f"{wl.name}: paced rows differ from the unpaced launch"


@pytest.mark.parametrize("types", TYPES, ids=lambda t: "-".join(t))
def test_paced_forced_splits(types):
    """20 sequences x 8 KV heads x 2 forced splits: 320 workgroups, paced,
    with partial states merged across workgroups (the last split of each
    pair merges).  Decode against the oracle on every row and bit-equal to
    the same sequences in an unpaced grid (the first 12: 192 workgroups);
    the one-launch step bit-equal to scatter + decode."""
    q, kv, new = types
    rng = np.random.default_rng(97)
    ctx = [int(c) for c in rng.integers(1500, 4001, size=20)]
    ctx[3], ctx[8] = 0, 17  # an empty sequence and one too short to pace
    wl = workloads.Workload(f"paced-splits-{q}-{kv}", 20, H_Q, H_KV, D, BS, q, kv, new, 97, contexts=tuple(ctx),
                            extra_blocks=9)
    print(f"[case] {wl.name} decode splits=2", flush=True)
    c = Case(wl)
    c.scatter()
    out = c.decode(num_splits=2)
    torch.cuda.synchronize()
    assert_close(out, c.oracle_decode(), wl.kv_dtype, label=f"{wl.name} all rows")
    sub = torch.empty((12, H_Q, D), dtype=torch.float32, device="cuda")
    ws = pkv.make_workspace(12, H_Q, H_KV, D, BS, c.plan.max_context_len, 2)
    pkv.pkv_paged_attention_decode(sub, c.t.q[:12].contiguous(), c.t.k_cache, c.t.v_cache,
                                   c.block_tables[:12].contiguous(), c.context_lens[:12].contiguous(),
                                   max_context_len=c.plan.max_context_len, k_scale=c.t.k_scale,
                                   v_scale=c.t.v_scale, num_splits=2, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(sub, out[:12]), f"{wl.name}: paced rows differ from the unpaced launch"

    print(f"[case] {wl.name} step splits=2", flush=True)
    two = Case(wl)
    two.scatter()
    ref_out = two.decode(num_splits=2)
    torch.cuda.synchronize()
    one = Case(wl)
    step_out = torch.empty_like(ref_out)
    pkv.pkv_decode_step(step_out, one.t.q, one.t.new_k, one.t.new_v, one.t.k_cache, one.t.v_cache, one.block_tables,
                        one.context_lens, max_context_len=one.plan.max_context_len, k_scale=one.t.k_scale,
                        v_scale=one.t.v_scale, num_splits=2)
    torch.cuda.synchronize()
    assert torch.equal(step_out, ref_out), f"{wl.name}: step output differs from scatter + decode"
    assert torch.equal(one.t.k_cache.view(torch.uint8), two.t.k_cache.view(torch.uint8)), f"{wl.name}: K pool"
    assert torch.equal(one.t.v_cache.view(torch.uint8), two.t.v_cache.view(torch.uint8)), f"{wl.name}: V pool"
