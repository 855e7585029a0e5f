"""Longest pairs first: when a decode grid of one workgroup per (sequence,
KV head, split) does not fit on the GPU at once, the library hands the
pairs to workgroups in decreasing order of their tile count (ties in index
order).  Which workgroup computes a pair changes nothing in its arithmetic,
so the output must equal, bit for bit, a call that forces the same split
count (forced counts keep the pairs in order), and both must match the
float64 oracle.
"""

import numpy as np
import pytest
import torch

import paged_kv_cache_431_amd as pkv
import workloads
from pkv_cases import Case, assert_close, to_bits

pytestmark = pytest.mark.gpu

RESIDENT_WORKGROUPS = 256 * 3  # one-workgroup-per-pair decode kernels: 3 per compute unit


def mixed(num_seqs, h_q, h_kv, d, q, kv, lens, seed):
    name = f"order-{q}-{kv}-s{num_seqs}-hq{h_q}-hkv{h_kv}-d{d}"
    return workloads.Workload(name, num_seqs, h_q, h_kv, d, 16, q, kv, q, seed, contexts=tuple(int(x) for x in lens),
                              extra_blocks=3)


def check_order(wl):
    print(f"[case] {wl.name}", flush=True)
    c = Case(wl)
    c.scatter()
    n = pkv.pkv_decode_num_splits(wl.num_seqs, wl.h_q, wl.h_kv, wl.head_dim, wl.block_size,
                                  c.plan.max_context_len, 0)
    grid = -(-wl.num_seqs * wl.h_kv // 8) * 8 * n
    assert grid > RESIDENT_WORKGROUPS, "the case must not fit on the GPU at once"
    ordered = c.decode(num_splits=0)
    in_order = c.decode(num_splits=n)
    torch.cuda.synchronize()
    assert np.array_equal(to_bits(ordered), to_bits(in_order)), f"{wl.name}: longest-first output differs"
    assert_close(ordered, c.oracle_decode(), wl.kv_dtype, label=f"{wl.name} splits={n}")


@pytest.mark.parametrize("types", [("bf16", "bf16"), ("f16", "f16"), ("bf16", "fp8")], ids=lambda t: "-".join(t))
@pytest.mark.parametrize("d", [64, 128])
def test_mixed_lengths_longest_first(types, d):
    """300 sequences x 8 KV heads (2,400 workgroups), lengths 0 ... 600 with
    empty and one-token sequences and many ties."""
    rng = np.random.default_rng(4310 + d)
    lens = rng.integers(0, 600, size=300, endpoint=True)
    lens[:7] = (0, 1, 16, 17, 0, 600, 1)
    check_order(mixed(300, 32, 8, d, *types, lens, seed=21))


def test_coarse_bins_for_long_contexts():
    """One 40,000-token sequence among 199 short ones: 2,500 tiles need
    coarser bins (tile counts halved), and the split count exceeds one."""
    rng = np.random.default_rng(4311)
    lens = rng.integers(0, 300, size=200, endpoint=True)
    lens[117] = 40000
    lens[3] = 32768
    check_order(mixed(200, 32, 8, 128, "bf16", "bf16", lens, seed=22))


def test_equal_lengths_keep_their_order():
    """All sequences alike: every rank is its own sequence."""
    check_order(mixed(120, 64, 8, 128, "bf16", "bf16", [300] * 120, seed=23))


def check_order_multi(wl, ms):
    """Several new query tokens per sequence: the same comparison."""
    print(f"[case] {wl.name} multi new<={max(ms)}", flush=True)
    c = Case(wl)
    c.scatter()
    q, qs = workloads.multi_queries(wl, ms, device="cuda")
    mq = max(max(ms), 1)
    n = pkv.pkv_multi_num_splits(wl.num_seqs, wl.h_q, wl.h_kv, wl.head_dim, wl.block_size, mq,
                                 c.plan.max_context_len, 0)
    ordered = c.multi(q, qs, mq, num_splits=0)
    in_order = c.multi(q, qs, mq, num_splits=n)
    torch.cuda.synchronize()
    assert np.array_equal(to_bits(ordered), to_bits(in_order)), f"{wl.name}: longest-first output differs"
    assert_close(ordered, c.oracle_multi(q, qs), wl.kv_dtype, label=f"{wl.name} multi splits={n}")


@pytest.mark.parametrize("group,tokens", [(4, 4), (8, 4), (8, 1), (8, 8)], ids=lambda x: str(x))
def test_multi_token_longest_first(group, tokens):
    """Speculative steps over 260 mixed-length sequences: one row tile per
    unit (4 x 4 rows), two row tiles held by one workgroup (8 x 4 rows), one
    token (decode rows through the multi-token kernel), and two row groups
    per unit (8 x 8 rows).  Some sequences have fewer cached tokens than new
    ones."""
    rng = np.random.default_rng(4312 + group + tokens)
    lens = rng.integers(1, 500, size=260, endpoint=True)
    lens[:4] = (1, 2, 3, 17)
    ms = np.minimum(tokens, lens)
    ms[1:3] = tokens  # 2 and 3 cached tokens: with 4 new ones the first rows see nothing
    ms[5] = 0  # a sequence with no new token this step
    check_order_multi(mixed(260, 8 * group, 8, 128, "bf16", "bf16", lens, seed=24), ms)
