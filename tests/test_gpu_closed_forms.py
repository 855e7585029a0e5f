"""Closed forms of attention on the HIP path (through the C ABI): a zero
query, or keys that are all equal, make every score the same, so the softmax
weights are uniform and the output is the plain mean of V over the context
("KV cache and PagedAttention in serving", section "PagedAttention: virtual
memory for GPUs": paged attention is attention over the logical sequence).
The expected rows come from the float64 oracle on the same bits, and the
oracle rows themselves are checked against the mean of V gathered here by
slot, so both the kernel and the reference are held to the closed form."""

import numpy as np
import pytest
import torch

import workloads
from pkv_cases import Case, assert_close

pytestmark = pytest.mark.gpu

RAGGED = (0, 1, 15, 16, 17, 100, 257, 300)

# (q, kv, new dtypes, block size): the matrix-core path (16-bit and FP8 caches
# with 16-token blocks) and the vector path (fp32 caches; 16-bit caches with
# 7-token blocks)
PATHS = [("bf16", "bf16", "bf16", 16), ("f16", "fp8", "f16", 16), ("bf16", "fp8", "bf16", 32),
         ("f32", "f32", "f32", 16), ("bf16", "bf16", "bf16", 7)]


def _case(q, kv, new, bs, seed):
    wl = workloads.Workload(f"closed-{q}-{kv}-b{bs}", len(RAGGED), 16, 2, 128, bs, q, kv, new, seed,
                            contexts=RAGGED, extra_blocks=5)
    return Case(wl)


def _mean_of_v(c):
    """float64 [S, Hq, D]: the mean over t < ctx_s of V_s[kv head of g, t],
    gathered slot by slot from the pool on the GPU (0 for an empty context)."""
    wl = c.wl
    vc = c.t.v_cache
    if wl.kv_dtype == "fp8":
        vals = vc.view(torch.float8_e4m3fn).double() * c.t.v_scale
    else:
        vals = vc.double()
    G = wl.h_q // wl.h_kv
    out = np.zeros((wl.num_seqs, wl.h_q, wl.head_dim))
    for s, ctx in enumerate(c.plan.context_lens.tolist()):
        if ctx == 0:
            continue
        t = torch.arange(ctx, device=vc.device)
        blocks = c.block_tables[s].long()[t // wl.block_size]
        rows = vals[blocks, :, t % wl.block_size, :]          # [ctx, Hkv, D]
        mean = rows.mean(dim=0).cpu().numpy()                 # [Hkv, D]
        out[s] = np.repeat(mean, G, axis=0)
    return out


@pytest.mark.parametrize("q,kv,new,bs", PATHS)
def test_zero_query_gives_the_mean_of_v(q, kv, new, bs):
    c = _case(q, kv, new, bs, 81)
    print(f"[case] {c.wl.name} q = 0", flush=True)
    c.t.q.zero_()
    c.scatter()
    out = c.decode()
    torch.cuda.synchronize()
    ref = c.oracle_decode()
    mean = _mean_of_v(c)
    assert np.allclose(ref, mean, rtol=1e-12, atol=1e-12), "oracle differs from the mean of V"
    assert_close(out, ref, kv, label=f"{c.wl.name} q=0")
    assert_close(out, mean, kv, label=f"{c.wl.name} q=0 vs mean")


@pytest.mark.parametrize("q,kv,new,bs", PATHS)
def test_equal_keys_give_the_mean_of_v(q, kv, new, bs):
    """Every cached key of a KV head, the new token's included, is one row:
    scores are equal whatever the query."""
    c = _case(q, kv, new, bs, 83)
    print(f"[case] {c.wl.name} equal keys", flush=True)
    wl = c.wl
    # every sequence's new token takes the key of the first one; the scatter
    # stores that one row (bits, or the FP8 codes it rounds to) in every new
    # token's slot, and the row is then copied into every slot of the pool
    c.t.new_k.copy_(c.t.new_k[:1].expand_as(c.t.new_k))
    c.scatter()
    s0 = next(s for s, ctx in enumerate(c.plan.context_lens.tolist()) if ctx >= 1)
    slot = int(c.rp.slot_mapping[s0])
    kc = c.t.k_cache
    row = kc[slot // wl.block_size, :, slot % wl.block_size, :].clone()   # [Hkv, D] as stored
    for sl in c.rp.slot_mapping.tolist():
        if sl >= 0:
            assert torch.equal(kc[sl // wl.block_size, :, sl % wl.block_size, :], row), "new tokens differ"
    kc.copy_(row[None, :, None, :].expand_as(kc))
    out = c.decode()
    torch.cuda.synchronize()
    ref = c.oracle_decode()
    mean = _mean_of_v(c)
    assert np.allclose(ref, mean, rtol=1e-12, atol=1e-12), "oracle differs from the mean of V"
    assert_close(out, ref, kv, label=f"{c.wl.name} equal keys")
    assert_close(out, mean, kv, label=f"{c.wl.name} equal keys vs mean")
