"""Pins of oracle.copy.swap_blocks (preemption by swapping).

  * End to end: a sequence's blocks are swapped out to a host pool, its
    device blocks are freed and reused by another sequence that writes its
    own tokens into them, then the sequence is admitted again into whatever
    blocks the allocator hands out and swapped back in.  Its paged attention
    afterwards equals its paged attention before preemption bit for bit, and
    the other sequence's attention equals plain float64 attention (torch
    SDPA) over its own tokens.
  * The move copies whole blocks (every head, every slot, K and V) and
    touches nothing else: checked through a flat slot view.
  * Calls with a repeated destination or an id outside its pool are
    rejected.
  * Planted mistakes (only K moved, only the first head moved, blocks moved
    one place off) fail the end-to-end pin.
"""

import numpy as np
import pytest
import torch

from oracle import allocator as al
from oracle import attention as att
from oracle import copy as cp
from oracle import scatter as sc


def _sdpa(q, k, v):
    G = q.shape[0] // k.shape[0]
    qt = torch.from_numpy(q)[:, None, :]
    kt = torch.from_numpy(k).repeat_interleave(G, dim=0)
    vt = torch.from_numpy(v).repeat_interleave(G, dim=0)
    return torch.nn.functional.scaled_dot_product_attention(qt[None], kt[None], vt[None])[0, :, 0, :].numpy()


def _write(bm, seq, kc, vc, toks_k, toks_v, bs):
    slots, _ = bm.append(seq, toks_k.shape[0])
    return sc.reshape_and_cache(toks_k.view(np.uint32), toks_v.view(np.uint32), kc, vc, slots,
                                in_dtype="f32", kv_dtype="f32", block_size=bs)


def _decode_one(q, kc, vc, table, n, bs):
    bt = np.array([table], dtype=np.int32)
    return att.paged_attention_decode(q[None].view(np.uint32), kc, vc, bt, np.array([n], dtype=np.int32),
                                      q_dtype="f32", kv_dtype="f32", block_size=bs)[0]


def preemption_round_trip_holds(len_a, len_c, swap_fn=cp.swap_blocks, seed=0):
    rng = np.random.default_rng(seed + 100 * len_a + len_c)
    bs, h_kv, h_q, d = 4, 2, 4, 8
    b_a, b_c = -(-len_a // bs), -(-len_c // bs)
    nb = b_a + b_c                                   # room for A and C at once, no more
    bm = al.BlockManager(nb, bs, free_order=rng.permutation(nb))
    kc = rng.standard_normal((nb, h_kv, bs, d)).astype(np.float32).view(np.uint32)
    vc = rng.standard_normal((nb, h_kv, bs, d)).astype(np.float32).view(np.uint32)
    bm.append(9, len_c)                              # a filler holds C's share first
    a_k = rng.standard_normal((len_a, h_kv, d)).astype(np.float32)
    a_v = rng.standard_normal((len_a, h_kv, d)).astype(np.float32)
    kc, vc = _write(bm, 0, kc, vc, a_k, a_v, bs)
    q_a = rng.standard_normal((h_q, d)).astype(np.float32)
    table_a, n_a = bm.block_table(0)
    before = _decode_one(q_a, kc, vc, table_a, n_a, bs)

    # preempt A: its blocks go to host blocks 0..len-1, then A (and the
    # filler) are freed, A's blocks first in the free list
    nh = b_a + 2
    hk = np.zeros((nh, h_kv, bs, d), dtype=np.uint32)
    hv = np.zeros((nh, h_kv, bs, d), dtype=np.uint32)
    hk, hv = swap_fn(hk, hv, kc, vc, [[b, j] for j, b in enumerate(table_a)])
    bm.free_seq(0)
    bm.free_seq(9)

    # C runs meanwhile and writes its tokens into A's freed blocks first
    c_k = rng.standard_normal((len_c, h_kv, d)).astype(np.float32)
    c_v = rng.standard_normal((len_c, h_kv, d)).astype(np.float32)
    kc, vc = _write(bm, 1, kc, vc, c_k, c_v, bs)
    table_c, n_c = bm.block_table(1)
    assert set(table_c) & set(table_a), "C must reuse a block A held"

    # A comes back into the blocks still free; its K/V are swapped in
    bm.append(2, len_a)
    table_a2, n_a2 = bm.block_table(2)
    assert n_a2 == len_a and not set(table_a2) & set(table_c)
    kc2, vc2 = swap_fn(kc, vc, hk, hv, [[j, b] for j, b in enumerate(table_a2)])
    after = _decode_one(q_a, kc2, vc2, table_a2, n_a2, bs)

    # C, still running, is untouched by the swap-in
    q_c = rng.standard_normal((h_q, d)).astype(np.float32)
    got = _decode_one(q_c, kc2, vc2, table_c, n_c, bs)
    ref = _sdpa(q_c.astype(np.float64), c_k.transpose(1, 0, 2).astype(np.float64),
                c_v.transpose(1, 0, 2).astype(np.float64))
    return bool(np.array_equal(before, after) and np.allclose(got, ref, rtol=1e-12, atol=1e-12))


@pytest.mark.parametrize("len_a,len_c", [(5, 9), (13, 4), (16, 16), (1, 30), (27, 3)])
def test_preemption_by_swap_round_trip(len_a, len_c):
    assert preemption_round_trip_holds(len_a, len_c)


def test_swap_moves_whole_blocks_and_nothing_else():
    rng = np.random.default_rng(5)
    nb, nh, h_kv, bs, d = 9, 6, 3, 4, 5
    dk = rng.integers(0, 2 ** 16, (nb, h_kv, bs, d)).astype(np.uint16)
    dv = rng.integers(0, 2 ** 16, (nb, h_kv, bs, d)).astype(np.uint16)
    sk = rng.integers(0, 2 ** 16, (nh, h_kv, bs, d)).astype(np.uint16)
    sv = rng.integers(0, 2 ** 16, (nh, h_kv, bs, d)).astype(np.uint16)
    pairs = [[5, 0], [0, 8], [3, 3], [5, 4]]                  # a source may repeat
    ok_, ov_ = cp.swap_blocks(dk, dv, sk, sv, pairs)
    flat = lambda c: np.transpose(c, (0, 2, 1, 3)).reshape(-1, h_kv, d)
    fdk, fdv, fsk, fsv, fok, fov = map(flat, (dk, dv, sk, sv, ok_, ov_))
    moved = {dst: src for src, dst in pairs}
    for slot in range(nb * bs):
        b, o = divmod(slot, bs)
        if b in moved:
            assert np.array_equal(fok[slot], fsk[moved[b] * bs + o]) and np.array_equal(fov[slot], fsv[moved[b] * bs + o])
        else:
            assert np.array_equal(fok[slot], fdk[slot]) and np.array_equal(fov[slot], fdv[slot])


@pytest.mark.parametrize("pairs", [[[1, 2], [3, 2]], [[0, 9]], [[6, 0]], [[-1, 2]]])
def test_repeated_destination_or_out_of_range_rejected(pairs):
    dst = np.zeros((9, 1, 2, 2), np.float32)
    src = np.zeros((6, 1, 2, 2), np.float32)
    with pytest.raises(ValueError):
        cp.swap_blocks(dst, dst, src, src, pairs)


def _k_only(dk, dv, sk, sv, pairs):
    k, _ = cp.swap_blocks(dk, dv, sk, sv, pairs)
    return k, np.array(dv, copy=True)


def _first_head_only(dk, dv, sk, sv, pairs):
    k, v = np.array(dk, copy=True), np.array(dv, copy=True)
    for s, d in pairs:
        k[d, 0], v[d, 0] = sk[s, 0], sv[s, 0]
    return k, v


def _one_off(dk, dv, sk, sv, pairs):
    return cp.swap_blocks(dk, dv, sk, sv, [[s, (d + 1) % dk.shape[0]] for s, d in pairs])


@pytest.mark.parametrize("mutant", [_k_only, _first_head_only, _one_off], ids=lambda f: f.__name__)
def test_planted_swap_mistake_is_caught(mutant):
    assert not all(preemption_round_trip_holds(a, c, mutant) for a, c in ((5, 9), (13, 4), (16, 16)))
