"""Pins of oracle.scatter and oracle.allocator.

Allocator: the numbers the pages print (52 blocks / 7 unused slots for an
825-token request; 47 such requests in a 2,457-block pool and no 48th), the
invariants they state (tail waste <= block_size - 1, growth never relocates a
block, a block is free exactly when nothing references it, copy-on-write only
when a shared tail block is written), checked over random operation sequences.

Scatter: written bytes land where a flat slot view says they must, nothing
else changes, FP8 codes agree with PyTorch's own float8 cast, and the
composition allocator -> scatter -> paged attention equals plain attention
over the appended token sequence (float64 SDPA on the tokens in order).
"""

import numpy as np
import pytest
import torch

from oracle import allocator as al
from oracle import attention as att
from oracle import scatter as sc

# ---------------------------------------------------------------- allocator


def test_825_token_request_layout():
    bm = al.BlockManager(2457, 16)
    slots, cow = bm.append(0, 825)
    table, n = bm.block_table(0)
    assert len(table) == 52 and n == 825 and cow == (-1, -1)
    assert len(table) * 16 - n == 7
    assert slots == [table[t // 16] * 16 + t % 16 for t in range(825)]
    assert bm.num_free() == 2457 - 52


def test_47_requests_fit_and_48th_does_not():
    bm = al.BlockManager(2457, 16, free_order=np.random.default_rng(0).permutation(2457))
    for s in range(47):
        bm.append(s, 825)
    assert bm.num_free() == 2457 - 47 * 52
    before = (list(bm.free), list(bm.refcount))
    with pytest.raises(al.OutOfBlocks):
        bm.append(47, 825)
    assert (list(bm.free), list(bm.refcount)) == before   # all or nothing
    assert 47 not in bm.tables


def test_fifo_order_and_one_block_per_boundary():
    bm = al.BlockManager(6, 4, free_order=[5, 2, 0, 4, 1, 3])
    assert bm.append(9, 1)[0] == [5 * 4]
    assert bm.append(9, 3)[0] == [21, 22, 23]
    assert bm.num_free() == 5
    assert bm.append(9, 1)[0] == [2 * 4]                  # 5th token claims the next free block
    assert bm.block_table(9) == ([5, 2], 5)


def test_fork_free_and_copy_on_write():
    bm = al.BlockManager(8, 4)
    bm.append(0, 6)                                        # blocks 0,1; block 1 half full
    bm.fork(0, 1)
    assert bm.refcount[0] == 2 and bm.refcount[1] == 2
    slots, cow = bm.append(1, 1)                           # child writes into the shared tail
    assert cow == (1, 2)
    assert slots == [2 * 4 + 2]
    assert bm.block_table(1) == ([0, 2], 7)
    assert bm.block_table(0) == ([0, 1], 6)                # parent untouched
    assert bm.refcount[1] == 1 and bm.refcount[2] == 1 and bm.refcount[0] == 2
    slots, cow = bm.append(0, 1)                           # parent's tail is no longer shared
    assert cow == (-1, -1) and slots == [1 * 4 + 2]
    bm.free_seq(0)                                         # block 0 still held by the child
    assert bm.refcount[0] == 1 and list(bm.free)[-1] == 1
    bm.free_seq(1)
    assert sorted(bm.free) == list(range(8))
    assert list(bm.free)[-2:] == [0, 2]                    # released in table order


def test_shared_full_prefix_needs_no_copy():
    bm = al.BlockManager(10, 4)
    bm.append(0, 8)                                        # two full blocks
    bm.fork(0, 1)
    slots, cow = bm.append(1, 1)
    assert cow == (-1, -1)
    assert bm.block_table(1)[0][:2] == [0, 1]


def test_invalid_requests():
    bm = al.BlockManager(4, 4)
    with pytest.raises(al.InvalidRequest):
        bm.append(-1, 1)
    with pytest.raises(al.InvalidRequest):
        bm.append(0, -1)
    with pytest.raises(al.InvalidRequest):
        bm.fork(3, 4)
    with pytest.raises(al.InvalidRequest):
        bm.free_seq(7)
    bm.append(0, 1)
    with pytest.raises(al.InvalidRequest):
        bm.fork(0, 0)
    with pytest.raises(al.InvalidRequest):
        al.BlockManager(4, 4, free_order=[0, 1, 1, 2])


def check_invariants(bm):
    bs = bm.block_size
    counted = [0] * bm.num_blocks
    for seq, table in bm.tables.items():
        n = bm.lengths[seq]
        assert len(table) == -(-n // bs)                   # tail waste <= bs - 1
        assert len(set(table)) == len(table)
        for b in table:
            counted[b] += 1
    assert counted == bm.refcount
    free = list(bm.free)
    assert len(set(free)) == len(free)
    assert set(free) == {b for b in range(bm.num_blocks) if bm.refcount[b] == 0}


@pytest.mark.parametrize("seed", range(6))
def test_random_operations_keep_invariants(seed):
    rng = np.random.default_rng(seed)
    bm = al.BlockManager(40, int(rng.choice([1, 2, 4, 16])), free_order=rng.permutation(40))
    live = []
    next_id = 0
    for _ in range(400):
        op = rng.integers(0, 10)
        if op < 6 or not live:
            seq = int(rng.choice(live)) if live and rng.random() < 0.8 else next_id
            before = bm.block_table(seq) if seq in bm.tables else ([], 0)
            try:
                slots, cow = bm.append(seq, int(rng.integers(0, 20)))
            except al.OutOfBlocks:
                check_invariants(bm)
                continue
            if seq == next_id:
                live.append(seq)
                next_id += 1
            table, n = bm.block_table(seq)
            keep = len(before[0]) - (1 if cow != (-1, -1) else 0)
            assert table[:keep] == before[0][:keep]        # growth never relocates
            if cow != (-1, -1):
                assert before[0][-1] == cow[0] and table[len(before[0]) - 1] == cow[1]
            bs = bm.block_size
            assert slots == [table[t // bs] * bs + t % bs for t in range(before[1], n)]
        elif op < 8:
            child = next_id
            bm.fork(int(rng.choice(live)), child)
            live.append(child)
            next_id += 1
        else:
            seq = int(rng.choice(live))
            bm.free_seq(seq)
            live.remove(seq)
        check_invariants(bm)

# ---------------------------------------------------------------- scatter


def test_scatter_same_dtype_writes_exact_bits_and_nothing_else():
    rng = np.random.default_rng(1)
    nb, h, bs, d = 7, 3, 4, 5
    kc = rng.integers(0, 2 ** 16, size=(nb, h, bs, d), dtype=np.uint16)
    vc = rng.integers(0, 2 ** 16, size=(nb, h, bs, d), dtype=np.uint16)
    key = rng.integers(0, 2 ** 16, size=(5, h, d), dtype=np.uint16)
    val = rng.integers(0, 2 ** 16, size=(5, h, d), dtype=np.uint16)
    slots = np.array([0, 27, -1, 13, 6], dtype=np.int64)
    k2, v2 = sc.reshape_and_cache(key, val, kc, vc, slots, in_dtype="bf16", kv_dtype="bf16", block_size=bs)
    flat_k = kc.transpose(0, 2, 1, 3).reshape(nb * bs, h, d).copy()
    flat_v = vc.transpose(0, 2, 1, 3).reshape(nb * bs, h, d).copy()
    for i, s in enumerate(slots):
        if s >= 0:
            flat_k[s] = key[i]
            flat_v[s] = val[i]
    assert np.array_equal(k2.transpose(0, 2, 1, 3).reshape(nb * bs, h, d), flat_k)
    assert np.array_equal(v2.transpose(0, 2, 1, 3).reshape(nb * bs, h, d), flat_v)


@pytest.mark.parametrize("in_dtype,tdtype", [("f32", torch.float32), ("bf16", torch.bfloat16), ("f16", torch.float16)])
def test_scatter_fp8_matches_library_cast(in_dtype, tdtype):
    rng = np.random.default_rng(2)
    x = torch.from_numpy(rng.standard_normal((6, 2, 16)).astype(np.float32) * 3).to(tdtype)
    y = torch.from_numpy(rng.standard_normal((6, 2, 16)).astype(np.float32)).to(tdtype)
    bits_dtype = {torch.float32: torch.int32, torch.bfloat16: torch.int16, torch.float16: torch.int16}[tdtype]
    np_bits = {torch.float32: np.uint32, torch.bfloat16: np.uint16, torch.float16: np.uint16}[tdtype]
    kb = x.view(bits_dtype).numpy().view(np_bits)
    vb = y.view(bits_dtype).numpy().view(np_bits)
    ks, vs = 0.0625, 0.01
    kc = np.zeros((3, 2, 4, 16), dtype=np.uint8)
    vc = np.zeros((3, 2, 4, 16), dtype=np.uint8)
    slots = np.array([0, 5, 11, 2, 7, 9], dtype=np.int64)
    k2, v2 = sc.reshape_and_cache(kb, vb, kc, vc, slots, in_dtype=in_dtype, kv_dtype="fp8", block_size=4,
                                  k_scale=ks, v_scale=vs)
    ref_k = (x.float() / torch.tensor(ks, dtype=torch.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ref_v = (y.float() / torch.tensor(vs, dtype=torch.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    for i, s in enumerate(slots):
        assert np.array_equal(k2[s // 4, :, s % 4, :], ref_k[i])
        assert np.array_equal(v2[s // 4, :, s % 4, :], ref_v[i])


def test_allocator_scatter_attention_compose_to_plain_attention():
    """Tokens appended through the block manager, scattered into a shuffled
    pool and attended through the block table give exactly the attention of
    the token sequence in order (the continuous-sequence view the pages
    describe)."""
    rng = np.random.default_rng(3)
    nb, h_q, h_kv, bs, d = 30, 4, 2, 4, 8
    bm = al.BlockManager(nb, bs, free_order=rng.permutation(nb))
    kc = np.full((nb, h_kv, bs, d), np.nan, dtype=np.float32)
    vc = np.full((nb, h_kv, bs, d), np.nan, dtype=np.float32)
    tokens_k = {0: [], 1: [], 2: []}
    tokens_v = {0: [], 1: [], 2: []}
    for step in range(40):
        seqs = [s for s in (0, 1, 2) if rng.random() < 0.7]
        if not seqs:
            continue
        key = rng.standard_normal((len(seqs), h_kv, d)).astype(np.float32)
        val = rng.standard_normal((len(seqs), h_kv, d)).astype(np.float32)
        slots = np.array([bm.append(s, 1)[0][0] for s in seqs], dtype=np.int64)
        kc_b, vc_b = sc.reshape_and_cache(key.view(np.uint32), val.view(np.uint32), kc.view(np.uint32),
                                          vc.view(np.uint32), slots, in_dtype="f32", kv_dtype="f32", block_size=bs)
        kc, vc = kc_b.view(np.float32), vc_b.view(np.float32)
        for i, s in enumerate(seqs):
            tokens_k[s].append(key[i])
            tokens_v[s].append(val[i])
    mb = max(len(bm.block_table(s)[0]) for s in (0, 1, 2))
    bt = np.full((3, mb), -1, dtype=np.int32)
    ctx = np.zeros(3, dtype=np.int32)
    for s in (0, 1, 2):
        table, n = bm.block_table(s)
        bt[s, :len(table)] = table
        ctx[s] = n
    q = rng.standard_normal((3, h_q, d)).astype(np.float32)
    out = att.paged_attention_decode(q.view(np.uint32), kc.view(np.uint32), vc.view(np.uint32), bt, ctx,
                                     q_dtype="f32", kv_dtype="f32", block_size=bs)
    for s in (0, 1, 2):
        k = torch.from_numpy(np.stack(tokens_k[s]).astype(np.float64)).permute(1, 0, 2).repeat_interleave(2, 0)
        v = torch.from_numpy(np.stack(tokens_v[s]).astype(np.float64)).permute(1, 0, 2).repeat_interleave(2, 0)
        qq = torch.from_numpy(q[s].astype(np.float64))[:, None, :]
        ref = torch.nn.functional.scaled_dot_product_attention(qq[None], k[None], v[None])[0, :, 0].numpy()
        assert np.allclose(out[s], ref, rtol=1e-12, atol=1e-12)
