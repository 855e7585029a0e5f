"""Decode with balanced ranges (few (sequence, KV head) pairs, long and
uneven contexts: the tiles of all pairs are cut into equal ranges, one per
workgroup) against the float64 oracle, through the C ABI:

  * ragged contexts with empty sequences, short ones that fit inside one
    range and long ones split over many workgroups, in 16-bit and FP8 pools;
  * the one-launch decode step gives the same bits as the scatter followed
    by decode, and the same pools;
  * 512 sequences of one KV head each (the most pairs the mode takes), so
    the prefix of tile counts spans many lanes;
  * repeated calls reuse the workspace (its counters return to zero);
  * contexts longer than max_context_len are attended over in full;
  * several new query tokens per sequence whose rows of a pair fit one
    workgroup take balanced ranges too (one and two row tiles, ragged
    token counts including none);
  * 16-bit outputs are the fp32 outputs rounded, from both merges.
"""

import numpy as np
import pytest
import torch

import paged_kv_cache_431_amd as pkv
import workloads
from pkv_cases import Case, assert_close, to_bits

pytestmark = pytest.mark.gpu

MIXED = (0, 1, 4096, 17, 8000, 0, 300, 12000, 16, 4097)


def _wl(name, contexts, kv="bf16", h_q=16, h_kv=2, bs=16, seed=91):
    q = "bf16" if kv in ("bf16", "fp8") else kv
    return workloads.Workload(name, len(contexts), h_q, h_kv, 128, bs, q, kv, q, seed, contexts=tuple(contexts),
                              extra_blocks=5)


def _step(c):
    wl = c.wl
    out = torch.empty((wl.num_seqs, wl.h_q, wl.head_dim), dtype=torch.float32, device="cuda")
    pkv.pkv_decode_step(out, c.t.q, c.t.new_k, c.t.new_v, c.t.k_cache, c.t.v_cache, c.block_tables,
                        c.context_lens, max_context_len=c.plan.max_context_len, k_scale=c.t.k_scale,
                        v_scale=c.t.v_scale)
    return out


@pytest.mark.parametrize("kv", ["bf16", "f16", "fp8"])
def test_balanced_ranges_match_the_oracle(kv):
    wl = _wl(f"balanced-{kv}", MIXED, kv=kv)
    print(f"[case] {wl.name}", flush=True)
    c = Case(wl)
    c.scatter()
    out = c.decode()
    torch.cuda.synchronize()
    assert_close(out, c.oracle_decode(), wl.kv_dtype, label=wl.name)
    again = c.decode()
    torch.cuda.synchronize()
    assert torch.equal(out, again), "a second call on the same workspace differs"

    print(f"[case] {wl.name} decode step", flush=True)
    one = Case(wl)
    got = _step(one)
    torch.cuda.synchronize()
    assert torch.equal(got, out), "decode step differs from scatter + decode"
    assert np.array_equal(to_bits(one.t.k_cache), to_bits(c.t.k_cache))
    assert np.array_equal(to_bits(one.t.v_cache), to_bits(c.t.v_cache))


def test_balanced_and_split_assignments_agree():
    """The same inputs through balanced ranges (library's choice) and through
    forced splits (one workgroup per pair and split): both within tolerance
    of the oracle, and of each other."""
    wl = _wl("balanced-vs-splits", MIXED, seed=93)
    c = Case(wl)
    c.scatter()
    ref = c.oracle_decode()
    for splits in (0, 3):
        print(f"[case] {wl.name} splits={splits}", flush=True)
        out = c.decode(num_splits=splits)
        torch.cuda.synchronize()
        assert_close(out, ref, wl.kv_dtype, label=f"{wl.name}-splits{splits}")


def test_most_pairs_the_balanced_mode_takes():
    rng = np.random.default_rng(95)
    contexts = rng.integers(0, 5000, 512)
    contexts[:3] = (4999, 0, 1)
    wl = _wl("balanced-512", tuple(int(x) for x in contexts), h_q=8, h_kv=1, seed=97)
    print(f"[case] {wl.name}", flush=True)
    c = Case(wl)
    c.scatter()
    out = c.decode()
    torch.cuda.synchronize()
    seqs = sorted(set(rng.choice(wl.num_seqs, 24, replace=False).tolist()) | {0, 1, 2, wl.num_seqs - 1})
    assert_close(out, c.oracle_decode(seqs=seqs), wl.kv_dtype, seqs=seqs, label=wl.name)
    assert torch.isfinite(out).all()
    assert torch.count_nonzero(out[1]) == 0, "a sequence with no context must get zeros"


def test_contexts_beyond_max_context_len_are_exact():
    """max_context_len only sizes the assignment: sequences longer than it
    (within their block tables) are still attended over in full, with
    balanced ranges as with one workgroup per pair and split."""
    wl = _wl("balanced-long-tail", (9000, 300, 4500, 0, 12000, 17), seed=99)
    c = Case(wl)
    c.scatter()
    ref = c.oracle_decode()
    short = 5000  # still long enough for balanced ranges (313 tiles)
    assert c.plan.max_context_len > short
    for splits in (0, 2):
        print(f"[case] {wl.name} max_context_len={short} splits={splits}", flush=True)
        ws = pkv.make_workspace(wl.num_seqs, wl.h_q, wl.h_kv, wl.head_dim, wl.block_size, short, splits)
        out = torch.empty((wl.num_seqs, wl.h_q, wl.head_dim), dtype=torch.float32, device="cuda")
        pkv.pkv_paged_attention_decode(out, c.t.q, c.t.k_cache, c.t.v_cache, c.block_tables, c.context_lens,
                                       max_context_len=short, k_scale=c.t.k_scale, v_scale=c.t.v_scale,
                                       num_splits=splits, workspace=ws)
        torch.cuda.synchronize()
        assert_close(out, ref, wl.kv_dtype, label=f"{wl.name}-splits{splits}")


# several new query tokens per sequence whose rows of a pair fit one
# workgroup (m x group <= 32): balanced ranges as for decode
@pytest.mark.parametrize("kv,h_q,ms", [("bf16", 16, (1, 4, 2, 3, 0, 4, 1, 2, 4, 3)),     # group 8: two row tiles
                                       ("fp8", 16, (4, 1, 3, 4, 4, 2, 1, 0, 3, 4)),
                                       ("f16", 8, (1, 2, 4, 3, 4, 1, 2, 4, 0, 4)),       # group 4: one row tile
                                       ("fp8", 4, (8, 1, 3, 8, 5, 2, 8, 1, 3, 6))])      # group 2, m up to 8
def test_balanced_ranges_with_several_query_tokens(kv, h_q, ms):
    wl = _wl(f"balanced-multi-{kv}-hq{h_q}", MIXED, kv=kv, h_q=h_q, seed=101)
    max_m = max(ms)
    assert max_m * wl.group <= 32
    # the library takes balanced ranges for this call
    assert pkv.pkv_multi_num_splits(wl.num_seqs, wl.h_q, wl.h_kv, wl.head_dim, wl.block_size, max_m,
                                    max(MIXED)) > 3
    print(f"[case] {wl.name} new={ms}", flush=True)
    c = Case(wl)
    c.scatter()
    q, qs = workloads.multi_queries(wl, ms, device="cuda")
    out = c.multi(q, qs, max_m)
    torch.cuda.synchronize()
    ref = c.oracle_multi(q, qs)
    assert_close(out, ref, wl.kv_dtype, label=wl.name)
    again = c.multi(q, qs, max_m)
    torch.cuda.synchronize()
    assert torch.equal(out, again), "a second call on the same workspace differs"
    # one workgroup per pair and split: the same result within tolerance
    forced = c.multi(q, qs, max_m, num_splits=3)
    torch.cuda.synchronize()
    assert_close(forced, ref, wl.kv_dtype, label=f"{wl.name}-splits3")


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float16])
def test_balanced_ranges_16bit_output_is_the_rounded_fp32_output(out_dtype):
    """Short sequences that fit inside one range write their rows from the
    workgroup's own merge (consecutive elements per thread), long ones from
    the cross-range merge (every 16th element): both round the fp32 output
    to nearest-even, for decode and for several query tokens."""
    wl = _wl("balanced-out16", MIXED, kv="bf16", seed=103)
    c = Case(wl)
    c.scatter()
    f32 = c.decode()
    o16 = c.decode(out_dtype=out_dtype)
    torch.cuda.synchronize()
    assert torch.equal(o16, f32.to(out_dtype))
    ms = (1, 4, 2, 3, 0, 4, 1, 2, 4, 3)
    q, qs = workloads.multi_queries(wl, ms, device="cuda")
    m32 = c.multi(q, qs, max(ms))
    m16 = c.multi(q, qs, max(ms), out_dtype=out_dtype)
    torch.cuda.synchronize()
    assert torch.equal(m16, m32.to(out_dtype))
