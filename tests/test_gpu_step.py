"""The one-launch decode step (the new tokens' scatter inside the decode
kernel) through the C ABI: the same output bits and the same pool bytes as
the scatter followed by decode on identical seeded inputs, and the oracle's
result within the decode tolerances.  The new tokens' slots start poisoned
(NaN), so a step that attended over the stale slot could not match."""

import numpy as np
import pytest
import torch

import paged_kv_cache_431_amd as pkv
import workloads
from pkv_cases import Case, assert_close, to_bits

pytestmark = pytest.mark.gpu

RAGGED = (0, 1, 15, 16, 17, 100, 257, 300)
MFMA_TYPES = [("bf16", "bf16", "bf16"), ("f16", "f16", "f16"), ("bf16", "fp8", "bf16"), ("f16", "fp8", "f16"),
              ("bf16", "fp8", "f32")]


def small(h_q, h_kv, d, bs, q, kv, new, contexts=RAGGED, seed=51):
    name = f"step-{q}-{kv}-{new}-hq{h_q}-hkv{h_kv}-d{d}-b{bs}"
    return workloads.Workload(name, len(contexts), h_q, h_kv, d, bs, q, kv, new, seed, contexts=tuple(contexts),
                              extra_blocks=5)


def step(c, num_splits=0, out_dtype=torch.float32):
    wl = c.wl
    out = torch.empty((wl.num_seqs, wl.h_q, wl.head_dim), dtype=out_dtype, device="cuda")
    pkv.pkv_decode_step(out, c.t.q, c.t.new_k, c.t.new_v, c.t.k_cache, c.t.v_cache, c.block_tables, c.context_lens,
                        max_context_len=c.plan.max_context_len, k_scale=c.t.k_scale, v_scale=c.t.v_scale,
                        num_splits=num_splits)
    return out


def check_step(wl, num_splits=0, oracle_seqs=None, label=None):
    label = label or wl.name
    print(f"[case] {label} splits={num_splits}", flush=True)
    two = Case(wl)
    two.scatter()
    ref_out = two.decode(num_splits=num_splits)
    one = Case(wl)
    out = step(one, num_splits)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out), f"{label}: step output differs from scatter + decode"
    assert torch.equal(one.t.k_cache.view(torch.uint8), two.t.k_cache.view(torch.uint8)), f"{label}: K pool"
    assert torch.equal(one.t.v_cache.view(torch.uint8), two.t.v_cache.view(torch.uint8)), f"{label}: V pool"
    ref = one.oracle_decode(seqs=oracle_seqs)
    rows = oracle_seqs
    assert_close(out, ref, wl.kv_dtype, seqs=rows, label=label)


@pytest.mark.parametrize("types", MFMA_TYPES, ids=lambda t: "-".join(t))
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("group", [1, 8, 16])
@pytest.mark.parametrize("bs", [16, 32])
def test_step_equals_scatter_then_decode(types, d, group, bs):
    check_step(small(2 * group, 2, d, bs, *types))


@pytest.mark.parametrize("splits", [1, 2, 3, 5, 16])
@pytest.mark.parametrize("types", [("bf16", "bf16", "bf16"), ("bf16", "fp8", "bf16")], ids=lambda t: "-".join(t))
def test_step_with_forced_splits(splits, types):
    """The new token's tile is in the last split; many splits leave it to a
    workgroup whose waves hold one tile or none."""
    wl = small(16, 2, 128, 16, *types, contexts=(1, 33, 250, 600, 1000, 7, 0, 511), seed=53)
    check_step(wl, num_splits=splits, label=f"{wl.name}-splits{splits}")


@pytest.mark.parametrize("name", ["gqa70b-bf16-47x825", "fp8-prefix-32xU32768"])
def test_step_on_named_workload(name):
    wl = workloads.get(name)
    rng = np.random.default_rng(55)
    seqs = sorted(set(rng.choice(wl.num_seqs, 4, replace=False).tolist()))
    check_step(wl, oracle_seqs=seqs, label=name)


def test_fp32_cache_is_unsupported():
    c = Case(small(8, 2, 64, 16, "f32", "f32", "f32", contexts=(20, 5)))
    with pytest.raises(pkv.PkvError, match="PKV_EUNSUPPORTED"):
        step(c)
