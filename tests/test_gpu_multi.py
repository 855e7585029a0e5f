"""Parity of the HIP path for several new query tokens per sequence (causal),
through the C ABI, with the float64 oracle.

Each test scatters the decode step's new tokens into a poisoned pool (NaN in
every slot that holds no token, checked bit-exact against the oracle's
scatter), draws m_s query rows per sequence, and compares every output row
(sampled rows at full workload sizes) within max-abs 2e-2 (6e-2 for FP8) and
rel-L2 1e-3.
"""

import numpy as np
import pytest
import torch

import paged_kv_cache_431_amd as pkv
import workloads
from pkv_cases import Case, assert_close, to_bits

pytestmark = pytest.mark.gpu

CONTEXTS = (1, 15, 16, 17, 100, 257, 300)
NEW = (1, 2, 16, 17, 5, 33, 3)      # ctx = m: a whole prompt; 17 and 33: ragged row tiles


def small(h_q, h_kv, d, bs, q, kv, new, contexts=CONTEXTS, seed=21):
    name = f"multi-{q}-{kv}-hq{h_q}-hkv{h_kv}-d{d}-b{bs}"
    return workloads.Workload(name, len(contexts), h_q, h_kv, d, bs, q, kv, new, seed, contexts=tuple(contexts),
                              extra_blocks=5)


def prepared(wl):
    c = Case(wl)
    kc, vc = c.scatter()
    ko, vo = c.oracle_pools()
    assert np.array_equal(to_bits(kc), ko), f"{wl.name}: K pool differs after scatter"
    assert np.array_equal(to_bits(vc), vo), f"{wl.name}: V pool differs after scatter"
    return c


def check_multi(wl, ms, num_splits=0, label=None, out_dtype=torch.float32):
    label = label or wl.name
    print(f"[case] {label} new={tuple(ms)} splits={num_splits}", flush=True)
    c = prepared(wl)
    q, qs = workloads.multi_queries(wl, ms, device="cuda")
    out = c.multi(q, qs, max(max(ms), 1), out_dtype=out_dtype, num_splits=num_splits)
    torch.cuda.synchronize()
    ref = c.oracle_multi(q, qs)
    assert_close(out, ref, wl.kv_dtype, label=label)
    return c, q, qs, out, ref


MFMA_TYPES = [("bf16", "bf16", "bf16"), ("f16", "f16", "f16"), ("bf16", "fp8", "bf16"), ("f16", "fp8", "f16")]


@pytest.mark.parametrize("types", MFMA_TYPES, ids=lambda t: "-".join(t))
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("group", [1, 4, 8, 16])
@pytest.mark.parametrize("bs", [16, 32])
def test_matrix_core_multi(types, d, group, bs):
    check_multi(small(2 * group, 2, d, bs, *types), NEW)


@pytest.mark.parametrize("splits", [1, 2, 3, 7, 16])
@pytest.mark.parametrize("types", [("bf16", "bf16", "bf16"), ("bf16", "fp8", "bf16")], ids=lambda t: "-".join(t))
def test_forced_splits_multi(splits, types):
    wl = small(16, 2, 128, 16, *types, contexts=(1, 33, 250, 600, 1000, 7), seed=23)
    check_multi(wl, (1, 9, 4, 20, 2, 7), num_splits=splits, label=f"{wl.name}-splits{splits}")


def test_more_new_tokens_than_cached_ones():
    """Tokens before the first cached position attend over nothing: 0."""
    wl = small(8, 2, 128, 16, "bf16", "bf16", "bf16", contexts=(3, 0, 10, 40), seed=25)
    _, _, qs, out, ref = check_multi(wl, (5, 2, 12, 1))
    o = out.cpu().numpy()
    assert np.all(o[0:2] == 0) and np.all(o[5:7] == 0) and np.all(o[7:9] == 0)
    assert np.all(ref[0:2] == 0) and np.all(ref[5:7] == 0)


def test_one_new_token_is_bitwise_decode():
    """m_s = 1 and query_start = 0..S: the same launch as decode, same bits."""
    wl = small(16, 2, 128, 16, "bf16", "bf16", "bf16", seed=27)
    c = prepared(wl)
    dec = c.decode()
    qs = np.arange(wl.num_seqs + 1, dtype=np.int32)
    mul = c.multi(c.t.q, qs, 1)
    torch.cuda.synchronize()
    assert torch.equal(dec, mul)


def test_rows_outside_the_query_table_are_untouched():
    """m_s above max_query_len and offsets past T are clamped on the device:
    rows cut off keep their previous contents."""
    wl = small(8, 2, 128, 16, "bf16", "bf16", "bf16", contexts=(40, 30, 20), seed=29)
    c = prepared(wl)
    q, _ = workloads.multi_queries(wl, (4, 6, 2), device="cuda")        # T = 12 rows
    qs = np.array([0, 4, 10, 100], dtype=np.int32)                      # last offset past T
    out = torch.full((12, wl.h_q, wl.head_dim), 7.0, dtype=torch.float32, device="cuda")
    c.multi(q, qs, 4, out=out)                                          # seq 1 has 6 > 4 rows
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    assert np.all(o[8:10] == 7.0), "rows past max_query_len were written"
    # what the device computed: seq 1 = its first 4 rows treated as its only new tokens
    # (positions ctx - 4 + i), seq 2 = rows 10..11 (offset clamped to T = 12)
    ref_a = c.oracle_multi(q, np.array([0, 4, 8, 8], dtype=np.int32))
    ref_b = c.oracle_multi(q, np.array([0, 0, 10, 12], dtype=np.int32), seqs=[2])
    ref = np.concatenate([ref_a[:8], ref_b[10:12]])
    assert_close(torch.from_numpy(np.concatenate([o[:8], o[10:12]])), ref, "bf16", label="clamped rows")


def test_empty_query_table_is_a_no_op():
    wl = small(8, 2, 128, 16, "bf16", "bf16", "bf16", contexts=(40, 30), seed=31)
    c = prepared(wl)
    q = torch.empty((0, wl.h_q, wl.head_dim), dtype=torch.bfloat16, device="cuda")
    out = c.multi(q, np.zeros(3, dtype=np.int32), 1)
    torch.cuda.synchronize()
    assert out.shape[0] == 0


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float16])
def test_16bit_output_is_the_rounded_fp32_output(out_dtype, d):
    wl = small(16, 2, d, 16, "bf16", "bf16", "bf16", seed=33)
    c = prepared(wl)
    q, qs = workloads.multi_queries(wl, NEW, device="cuda")
    o32 = c.multi(q, qs, max(NEW))
    o16 = c.multi(q, qs, max(NEW), out_dtype=out_dtype)
    torch.cuda.synchronize()
    assert torch.equal(o32.to(out_dtype), o16)


def test_fp32_cache_is_unsupported():
    wl = small(8, 2, 64, 16, "f32", "f32", "f32", contexts=(20, 5), seed=35)
    c = prepared(wl)
    q, qs = workloads.multi_queries(wl, (2, 1), device="cuda")
    with pytest.raises(pkv.PkvError, match="PKV_EUNSUPPORTED"):
        c.multi(q, qs, 2)


@pytest.mark.parametrize("name,m", [("gqa70b-bf16-47x825", 4), ("fp8-prefix-32xU32768", 8)])
def test_speculative_step_on_named_workload(name, m):
    """m lookahead tokens per sequence on a full-size workload, in the launch
    configuration the library picks (on the 70B shape a paced grid of 376
    workgroups): every output row against the oracle on the 70B shape (about
    a second of oracle time), every row of sampled sequences (the longest,
    the shortest and random ones) on the 32K FP8 batch."""
    wl = workloads.get(name)
    c = Case(wl)
    c.scatter()
    ms = [m] * wl.num_seqs
    q, qs = workloads.multi_queries(wl, ms, device="cuda")
    out = c.multi(q, qs, m)
    torch.cuda.synchronize()
    if wl.num_seqs * m * wl.h_q * int(c.plan.context_lens.max()) <= 47 * 4 * 64 * 825:
        print(f"[case] {name} m={m} all rows", flush=True)
        assert_close(out, c.oracle_multi(q, qs), wl.kv_dtype, label=f"{name}-m{m} all rows")
        return
    ctx = c.plan.context_lens
    rng = np.random.default_rng(37)
    seqs = sorted({int(np.argmax(ctx)), int(np.argmin(ctx))} | set(rng.choice(wl.num_seqs, 3, replace=False).tolist()))
    print(f"[case] {name} m={m} sampled seqs {seqs}", flush=True)
    ref = c.oracle_multi(q, qs, seqs=seqs)
    rows = [r for s in seqs for r in range(int(qs[s]), int(qs[s + 1]))]
    assert_close(out, ref, wl.kv_dtype, seqs=rows, label=f"{name}-m{m}")
