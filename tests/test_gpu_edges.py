"""Edge cases of the boundary on the GPU, through the C ABI:

  * calls with nothing to do (no sequence, no token) succeed, launch nothing
    and leave every buffer as it was;
  * the scatter skips every slot outside the pool (a negative slot marks a
    padding token) and writes the others exactly as the oracle's scatter of
    the in-range tokens alone does, bit for bit over the whole pool;
  * block ids outside the pool and context lengths outside the table are
    kept inside their own sequence: the others keep their bits.
"""

import numpy as np
import pytest
import torch

import oracle.scatter
import paged_kv_cache_431_amd as pkv
import workloads
from pkv_cases import Case, to_bits

pytestmark = pytest.mark.gpu


def _case(kv):
    q = "bf16" if kv in ("bf16", "fp8") else kv
    wl = workloads.Workload(f"edges-{kv}", 6, 8, 2, 64, 16, q, kv, q, 71, contexts=(0, 1, 17, 40, 16, 33),
                            extra_blocks=3)
    return Case(wl)


@pytest.mark.parametrize("kv", ["bf16", "f32", "fp8"])
def test_empty_calls_touch_nothing(kv):
    c = _case(kv)
    wl = c.wl
    print(f"[case] {wl.name} empty calls", flush=True)
    k0, v0 = to_bits(c.t.k_cache).copy(), to_bits(c.t.v_cache).copy()
    mb = c.block_tables.shape[1]
    q0 = torch.empty((0, wl.h_q, wl.head_dim), dtype=c.t.q.dtype, device="cuda")
    out0 = torch.empty((0, wl.h_q, wl.head_dim), dtype=torch.float32, device="cuda")
    bt0 = torch.empty((0, mb), dtype=torch.int32, device="cuda")
    cl0 = torch.empty((0,), dtype=torch.int32, device="cuda")
    new0 = torch.empty((0, wl.h_kv, wl.head_dim), dtype=c.t.new_k.dtype, device="cuda")
    slots0 = torch.empty((0,), dtype=torch.int64, device="cuda")
    kw = dict(k_scale=c.t.k_scale, v_scale=c.t.v_scale)
    pkv.pkv_paged_attention_decode(out0, q0, c.t.k_cache, c.t.v_cache, bt0, cl0,
                                   max_context_len=c.plan.max_context_len, **kw)
    pkv.pkv_reshape_and_cache(new0, new0, c.t.k_cache, c.t.v_cache, slots0, **kw)
    if kv != "f32":  # the one-launch step exists for the matrix-core caches
        pkv.pkv_decode_step(out0, q0, new0, new0, c.t.k_cache, c.t.v_cache, bt0, cl0,
                            max_context_len=c.plan.max_context_len, **kw)
    torch.cuda.synchronize()
    assert np.array_equal(to_bits(c.t.k_cache), k0), "an empty call changed the K pool"
    assert np.array_equal(to_bits(c.t.v_cache), v0), "an empty call changed the V pool"


@pytest.mark.parametrize("kv", ["bf16", "f32", "fp8"])
def test_scatter_skips_slots_outside_the_pool(kv):
    c = _case(kv)
    wl = c.wl
    nb, bs = c.t.k_cache.shape[0], wl.block_size
    rng = np.random.default_rng(72)
    slots = rng.choice(nb * bs, size=wl.num_seqs, replace=False).astype(np.int64)
    slots[1] = -1                # padding
    slots[3] = nb * bs           # one past the pool
    slots[4] = nb * bs + 12345
    slots[5] = -(1 << 40)
    print(f"[case] {wl.name} slots {slots.tolist()}", flush=True)
    k0, v0 = to_bits(c.t.k_cache).copy(), to_bits(c.t.v_cache).copy()
    pkv.pkv_reshape_and_cache(c.t.new_k, c.t.new_v, c.t.k_cache, c.t.v_cache, torch.from_numpy(slots).cuda(),
                              k_scale=c.t.k_scale, v_scale=c.t.v_scale)
    torch.cuda.synchronize()
    keep = (slots >= 0) & (slots < nb * bs)
    assert keep.sum() == 2
    ek, ev = oracle.scatter.reshape_and_cache(
        to_bits(c.t.new_k)[keep], to_bits(c.t.new_v)[keep], k0.copy(), v0.copy(), slots[keep],
        in_dtype=wl.new_dtype, kv_dtype=wl.kv_dtype, block_size=bs, k_scale=c.t.k_scale, v_scale=c.t.v_scale)
    assert np.array_equal(to_bits(c.t.k_cache), ek), "K pool differs from the oracle's scatter of the in-range slots"
    assert np.array_equal(to_bits(c.t.v_cache), ev), "V pool differs from the oracle's scatter of the in-range slots"


@pytest.mark.parametrize("kv", ["bf16", "f32"])
def test_bad_device_data_stays_inside_its_sequence(kv):
    """Block ids outside the pool are skipped, a negative context length is
    taken as 0 and one beyond the table as the table's capacity: the call
    completes, the sequences with valid data keep their bits, and the one
    with a negative length gets zeros.  (What a sequence with bad ids
    receives is unspecified.)"""
    q = "bf16" if kv == "bf16" else kv
    c = Case(workloads.Workload(f"edges-bad-{kv}", 8, 8, 2, 64, 16, q, kv, q, 73,
                                contexts=(0, 1, 17, 40, 16, 33, 300, 77), extra_blocks=3))
    wl = c.wl
    good = [0, 1, 6, 7]
    c.scatter()
    clean = c.decode()
    nb, mb = c.t.k_cache.shape[0], c.block_tables.shape[1]
    bt = c.block_tables.clone()
    lens = c.context_lens.clone()
    bt[2, 0] = nb          # one past the pool
    bt[3, 1] = -7
    lens[4] = -5
    lens[5] = mb * wl.block_size + 1000
    print(f"[case] {wl.name} bad ids in sequences 2, 3; lengths {lens.tolist()}", flush=True)
    out = torch.empty_like(clean)
    pkv.pkv_paged_attention_decode(out, c.t.q, c.t.k_cache, c.t.v_cache, bt, lens,
                                   max_context_len=c.plan.max_context_len, k_scale=c.t.k_scale, v_scale=c.t.v_scale)
    torch.cuda.synchronize()
    for s in good:
        assert torch.equal(out[s], clean[s]), f"sequence {s} changed"
    assert torch.count_nonzero(out[4]) == 0, "a negative context length must give zeros"
    if kv != "f32":
        print(f"[case] {wl.name} decode step with the same tables", flush=True)
        k0, v0 = to_bits(c.t.k_cache).copy(), to_bits(c.t.v_cache).copy()
        out2 = torch.empty_like(clean)
        pkv.pkv_decode_step(out2, c.t.q, c.t.new_k, c.t.new_v, c.t.k_cache, c.t.v_cache, bt, lens,
                            max_context_len=c.plan.max_context_len, k_scale=c.t.k_scale, v_scale=c.t.v_scale)
        torch.cuda.synchronize()
        for s in good:
            assert torch.equal(out2[s], clean[s]), f"decode step: sequence {s} changed"
        assert torch.count_nonzero(out2[4]) == 0
        # the step rewrote the new tokens of the sequences with valid tables
        # at the slots they already held: those pools bytes are unchanged
        kb, vb = to_bits(c.t.k_cache), to_bits(c.t.v_cache)
        valid_blocks = c.rp.block_tables[good].ravel()
        valid_blocks = valid_blocks[(valid_blocks >= 0) & (valid_blocks < nb)]
        assert np.array_equal(kb[valid_blocks], k0[valid_blocks])
        assert np.array_equal(vb[valid_blocks], v0[valid_blocks])


@pytest.mark.parametrize("types", [("bf16", "bf16", "bf16"), ("bf16", "fp8", "bf16")], ids=lambda t: "-".join(t))
def test_step_writes_nothing_past_a_full_table(types):
    """A context length beyond the table's capacity is attended over the
    table's tokens, and the step writes no new token for it: position
    capacity - 1 holds a cached token of its own.  Sequence 0 fills its table
    exactly (5 blocks of 16); its length is raised past the table, and its
    blocks must keep every byte while the others take their new tokens as
    usual and keep their output bits."""
    q, kv, new = types
    c = Case(workloads.Workload(f"edges-full-{kv}", 4, 16, 2, 128, 16, q, kv, new, 74,
                                contexts=(80, 17, 33, 5), extra_blocks=4))
    wl = c.wl
    mb = c.block_tables.shape[1]
    assert mb * wl.block_size == 80 and (c.rp.block_tables[0] >= 0).all(), "sequence 0 fills its table"
    c.scatter()
    clean = c.decode()
    lens = c.context_lens.clone()
    lens[0] = 80 + 7
    print(f"[case] {wl.name} lengths {lens.tolist()} (capacity 80)", flush=True)
    k0, v0 = to_bits(c.t.k_cache).copy(), to_bits(c.t.v_cache).copy()
    out = torch.empty_like(clean)
    pkv.pkv_decode_step(out, c.t.q, c.t.new_k, c.t.new_v, c.t.k_cache, c.t.v_cache, c.block_tables, lens,
                        max_context_len=c.plan.max_context_len, k_scale=c.t.k_scale, v_scale=c.t.v_scale)
    torch.cuda.synchronize()
    # the other sequences rewrote their new tokens where the scatter had put
    # them, and sequence 0 wrote nothing: the pools are byte for byte as before
    assert np.array_equal(to_bits(c.t.k_cache), k0), "K pool changed"
    assert np.array_equal(to_bits(c.t.v_cache), v0), "V pool changed"
    # sequence 0 attends over its 80 cached tokens: decode's bits
    assert torch.equal(out, clean), "outputs differ from decode over the table's tokens"
