"""Parity of the HIP path (through the C ABI) with the float64 oracle.

Every test builds one decode step from seeded inputs: the new tokens'
K/V are scattered into a poisoned pool (NaN in every slot that holds no
token), then paged attention runs over it.  The scatter is checked
bit-exact over the whole pool, attention within max-abs 2e-2 (6e-2 for FP8)
and rel-L2 1e-3 of the float64 oracle.
"""

import numpy as np
import pytest
import torch

import workloads
from pkv_cases import Case, assert_close, to_bits

pytestmark = pytest.mark.gpu

RAGGED = (0, 1, 15, 16, 17, 100, 257, 300)


def small(h_q, h_kv, d, bs, q, kv, new, contexts=RAGGED, seed=7, extra=5):
    name = f"small-{q}-{kv}-hq{h_q}-hkv{h_kv}-d{d}-b{bs}"
    return workloads.Workload(name, len(contexts), h_q, h_kv, d, bs, q, kv, new, seed, contexts=tuple(contexts),
                              extra_blocks=extra)


def check_step(wl, num_splits=0, label=None):
    label = label or wl.name
    print(f"[case] {label} splits={num_splits}", flush=True)
    c = Case(wl)
    kc, vc = c.scatter()
    ko, vo = c.oracle_pools()
    assert np.array_equal(to_bits(kc), ko), f"{label}: K pool differs after scatter"
    assert np.array_equal(to_bits(vc), vo), f"{label}: V pool differs after scatter"
    out = c.decode(num_splits=num_splits)
    torch.cuda.synchronize()
    return c, out, assert_close(out, c.oracle_decode(), wl.kv_dtype, label=label)


MFMA_TYPES = [("bf16", "bf16", "bf16"), ("f16", "f16", "f16"), ("bf16", "fp8", "bf16"), ("f16", "fp8", "f16")]


@pytest.mark.parametrize("types", MFMA_TYPES, ids=lambda t: "-".join(t))
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("group", [1, 4, 8, 16])
@pytest.mark.parametrize("bs", [16, 32])
def test_matrix_core_path(types, d, group, bs):
    check_step(small(2 * group, 2, d, bs, *types))


# fp32 caches take the vector path at every block size; 16-bit and FP8 caches
# take it when the block size is not 16 times a power of two
VECTOR_CASES = [(types, bs) for types in [("f32", "f32", "f32"), ("bf16", "bf16", "bf16"), ("bf16", "fp8", "f32")]
                for bs in (1, 7, 16, 32) if types[1] == "f32" or bs % 16 != 0]


@pytest.mark.parametrize("types,bs", VECTOR_CASES, ids=lambda x: "-".join(x) if isinstance(x, tuple) else f"b{x}")
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("group", [1, 4, 16])
def test_vector_path(types, bs, d, group):
    check_step(small(2 * group, 2, d, bs, *types, contexts=(0, 1, 15, 16, 17, 40, 77)))


@pytest.mark.parametrize("types", [("bf16", "bf16", "bf16"), ("bf16", "fp8", "bf16"), ("f32", "f32", "f32")],
                         ids=lambda t: "-".join(t))
@pytest.mark.parametrize("splits", [1, 2, 3, 5, 16, 64])
@pytest.mark.parametrize("d", [64, 128])
def test_forced_splits(types, splits, d):
    """Few splits make every wave walk many tiles in a row (the accumulators
    carry across tiles); many splits leave waves with one tile or none."""
    wl = small(16, 2, d, 16, *types, contexts=(1, 33, 250, 600, 1000, 1023, 7, 511), seed=11)
    check_step(wl, num_splits=splits, label=f"{wl.name}-splits{splits}")


@pytest.mark.parametrize("name", sorted(workloads.NAMED))
def test_named_workload(name):
    """The pages' workloads at full size, in the bench's launch configuration:
    whole pools are compared after the scatter, and every output row of
    attention against the float64 oracle."""
    wl = workloads.get(name)
    print(f"[case] named {name}", flush=True)
    c = Case(wl)
    kc, vc = c.scatter()
    ko, vo = c.oracle_pools()
    assert np.array_equal(to_bits(kc), ko), f"{name}: K pool differs after scatter"
    assert np.array_equal(to_bits(vc), vo), f"{name}: V pool differs after scatter"
    out = c.decode()
    torch.cuda.synchronize()
    assert_close(out, c.oracle_decode_all(), wl.kv_dtype, label=f"{name} all rows")


def test_single_token_returns_its_value_exactly():
    wl = small(8, 2, 128, 16, "bf16", "bf16", "bf16", contexts=(1, 1, 1), seed=3)
    c = Case(wl)
    kc, vc = c.scatter()
    out = c.decode()
    v_new = c.t.new_v.float()                      # the only cached token is the new one
    expect = v_new.repeat_interleave(4, dim=1)     # each KV head serves 4 query heads
    assert torch.equal(out, expect)


def test_block_placement_and_unused_entries_do_not_change_bits():
    wl = small(32, 4, 128, 16, "bf16", "bf16", "bf16", contexts=(5, 300, 129, 64, 1000), seed=5, extra=40)
    c = Case(wl)
    c.scatter()
    base = c.decode()
    # move every physical block somewhere else and rewrite the tables to match
    nb = c.plan.num_blocks
    perm = torch.from_numpy(np.random.default_rng(9).permutation(nb)).to(c.device)
    kc2 = torch.empty_like(c.t.k_cache)
    vc2 = torch.empty_like(c.t.v_cache)
    kc2[perm] = c.t.k_cache
    vc2[perm] = c.t.v_cache
    bt = c.block_tables.clone()
    used = bt >= 0
    bt[used] = perm[bt[used].long()].int()
    # entries past each sequence's last block hold junk that must never be read
    bt[~used] = torch.randint(-2 ** 31, 2 ** 31 - 1, (int((~used).sum()),), dtype=torch.int32, device=c.device)
    moved = c.decode(block_tables=bt, k_cache=kc2, v_cache=vc2)
    assert torch.equal(base, moved)


def test_repeat_calls_are_bitwise_identical_and_workspace_is_reusable():
    wl = small(64, 8, 128, 16, "bf16", "bf16", "bf16", contexts=(825,) * 6 + (3000, 17), seed=13)
    c = Case(wl)
    c.scatter()
    import paged_kv_cache_431_amd as pkv
    ws = pkv.make_workspace(wl.num_seqs, wl.h_q, wl.h_kv, wl.head_dim, wl.block_size, c.plan.max_context_len)
    outs = [c.decode(workspace=ws) for _ in range(4)]
    for o in outs[1:]:
        assert torch.equal(outs[0], o)
    assert_close(outs[0], c.oracle_decode(), "bf16", label="repeat")


@pytest.mark.parametrize("d,kv", [(128, "bf16"), (64, "bf16"), (128, "f32"), (64, "f32")],
                         ids=["d128-mfma", "d64-mfma", "d128-vector", "d64-vector"])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float16])
def test_16bit_output_is_the_rounded_fp32_output(out_dtype, d, kv):
    """Each thread of the merge stores its elements of a row in 16-byte
    groups (two per row of 128, one per row of 64): every element of the
    16-bit output is the fp32 output rounded to nearest-even, on both paths."""
    q = "f32" if kv == "f32" else "bf16"
    wl = small(16, 2, d, 16, q, kv, kv, seed=17)
    c = Case(wl)
    c.scatter()
    f32 = c.decode()
    o16 = c.decode(out_dtype=out_dtype)
    assert torch.equal(o16, f32.to(out_dtype))


def test_split_count_changes_stay_within_tolerance():
    wl = small(64, 8, 128, 16, "bf16", "fp8", "bf16", contexts=(4000, 2500, 9000, 33), seed=19)
    c = Case(wl)
    c.scatter()
    ref = c.oracle_decode()
    for n in (1, 2, 7, 30):
        assert_close(c.decode(num_splits=n), ref, "fp8", label=f"splits={n}")


def test_units_not_a_multiple_of_the_compute_units():
    """300 units (75 sequences x 4 KV heads) of mixed lengths: more units
    than compute units, not a whole multiple of them; every output row."""
    rng = np.random.default_rng(23)
    contexts = tuple(int(c) for c in rng.integers(1, 300, size=75))
    wl = workloads.Workload("units-75x4", 75, 16, 4, 128, 16, "bf16", "bf16", "bf16", 29, contexts=contexts,
                            extra_blocks=7)
    check_step(wl, label="units-75x4")


def gqa70b_with_blocks_of(bs):
    """The 70B-shaped layer with blocks of bs tokens: the same 12 GiB budget
    per layer pool in blocks of another size (B is an engine and hardware
    choice, "Paged KV Cache" tutorial, "Freeze the Architecture and Memory
    Budget"; at 32 tokens each 825-token request takes 26 blocks)."""
    wl = workloads.get("gqa70b-bf16-47x825")
    return workloads.replace(wl, name=f"{wl.name}-b{bs}", block_size=bs,
                             num_blocks=wl.num_blocks * wl.block_size // bs)


def test_gqa70b_with_32_token_blocks():
    """Config of the headline at B = 32: whole pools after the scatter, every
    output row against the oracle."""
    wl = gqa70b_with_blocks_of(32)
    c, out, _ = check_step(wl, label=wl.name)
    assert c.block_tables.shape[1] == 26 and c.plan.num_blocks == 1228
