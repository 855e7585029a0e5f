"""K/V through the LDS ring.  The one-row-tile kernels over 16-bit caches
with head_dim 128 load their tiles straight into LDS when the grid needs
several rounds of three workgroups per CU (more than 768 workgroups), as the
8B-style and MHA batches do.  The cases here have such grids with mostly
short contexts, so the oracle stays quick:
  * ragged contexts whose last blocks' tail slots are NaN-poisoned (the ring
    must read them as zeros past the context, as the register ring does);
  * sequences long enough for several 64-tile chunks per wave;
  * the one-launch step (output and pools bit-equal to scatter + decode), with
    owners that hold one tile and owners whose last tile is in a later chunk
    than the one that loaded the new token's rows;
  * forced split counts (the owner in the last split, partial states merged);
  * several query tokens per sequence in one row tile.
Every output row is compared with the oracle."""

import pytest
import torch

import paged_kv_cache_431_amd as pkv
import workloads
from pkv_cases import Case, assert_close

pytestmark = pytest.mark.gpu

H_Q, H_KV, D = 32, 8, 128  # 100 sequences x 8 KV heads: 800 workgroups
SHORT = (0, 1, 15, 16, 17, 31, 33, 64, 100, 257)
TYPES = [("bf16", "bf16", "bf16"), ("f16", "f16", "f16")]


def contexts(num_seqs, long=(5000, 9000)):
    ctx = [SHORT[i % len(SHORT)] for i in range(num_seqs)]
    for i, c in enumerate(long):  # several 64-tile chunks per wave
        ctx[7 + 31 * i] = c
    return tuple(ctx)


def ring_case(types, bs, num_seqs=100, seed=61, tag=""):
    q, kv, new = types
    ctx = contexts(num_seqs)
    name = f"ring{tag}-{q}-{kv}-hq{H_Q}-hkv{H_KV}-b{bs}-s{num_seqs}"
    return workloads.Workload(name, num_seqs, H_Q, H_KV, D, bs, q, kv, new, seed, contexts=ctx, extra_blocks=5)


def step(c, num_splits=0):
    wl = c.wl
    out = torch.empty((wl.num_seqs, wl.h_q, wl.head_dim), dtype=torch.float32, device="cuda")
    pkv.pkv_decode_step(out, c.t.q, c.t.new_k, c.t.new_v, c.t.k_cache, c.t.v_cache, c.block_tables, c.context_lens,
                        max_context_len=c.plan.max_context_len, k_scale=c.t.k_scale, v_scale=c.t.v_scale,
                        num_splits=num_splits)
    return out


def check_step(wl, num_splits=0):
    print(f"[case] {wl.name} step splits={num_splits}", flush=True)
    two = Case(wl)
    two.scatter()
    ref_out = two.decode(num_splits=num_splits)
    torch.cuda.synchronize()
    one = Case(wl)
    out = step(one, num_splits)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out), f"{wl.name}: step output differs from scatter + decode"
    assert torch.equal(one.t.k_cache.view(torch.uint8), two.t.k_cache.view(torch.uint8)), f"{wl.name}: K pool"
    assert torch.equal(one.t.v_cache.view(torch.uint8), two.t.v_cache.view(torch.uint8)), f"{wl.name}: V pool"
    assert_close(out, one.oracle_decode(), wl.kv_dtype, label=f"{wl.name} step all rows")


@pytest.mark.parametrize("bs", [16, 32, 64])
@pytest.mark.parametrize("types", TYPES, ids=lambda t: "-".join(t))
def test_decode_through_the_lds_ring(types, bs):
    wl = ring_case(types, bs)
    print(f"[case] {wl.name} decode", flush=True)
    c = Case(wl)
    c.scatter()
    out = c.decode()
    torch.cuda.synchronize()
    assert_close(out, c.oracle_decode(), wl.kv_dtype, label=f"{wl.name} decode all rows")


@pytest.mark.parametrize("bs", [16, 32])
@pytest.mark.parametrize("types", TYPES, ids=lambda t: "-".join(t))
def test_step_through_the_lds_ring(types, bs):
    check_step(ring_case(types, bs, seed=63))


@pytest.mark.parametrize("splits", [2, 3])
def test_forced_splits_through_the_lds_ring(splits):
    """50 sequences x 8 KV heads x the forced split count: 800 or 1,200
    workgroups; the new token sits in the last split."""
    wl = ring_case(("bf16", "bf16", "bf16"), 16, num_seqs=50, seed=65, tag=f"-splits{splits}")
    check_step(wl, num_splits=splits)
    c = Case(wl)
    c.scatter()
    out = c.decode(num_splits=splits)
    torch.cuda.synchronize()
    assert_close(out, c.oracle_decode(), wl.kv_dtype, label=f"{wl.name} decode splits={splits}")


@pytest.mark.parametrize("types", TYPES, ids=lambda t: "-".join(t))
def test_several_query_tokens_through_the_lds_ring(types):
    """Up to 4 new tokens of 4 query heads each: one 16-row tile per (sequence,
    KV head), 800 workgroups; ragged token counts, one more than the cached
    tokens included."""
    wl = ring_case(types, 16, seed=67, tag="-multi")
    ms = [(1, 2, 3, 4, 0)[i % 5] for i in range(wl.num_seqs)]
    ms[1] = 2  # a sequence of one cached token with two new ones
    print(f"[case] {wl.name} new tokens", flush=True)
    c = Case(wl)
    c.scatter()
    q, qs = workloads.multi_queries(wl, ms, device="cuda")
    out = c.multi(q, qs, max(ms))
    torch.cuda.synchronize()
    assert_close(out, c.oracle_multi(q, qs), wl.kv_dtype, label=f"{wl.name} several tokens")
