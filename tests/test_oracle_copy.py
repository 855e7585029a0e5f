"""Pins of oracle.copy (the copy-on-write block copy).

  * End to end: a parent sequence with a partly filled last block is forked;
    the child appends one token, the allocator moves it onto a fresh block
    and reports (src, dst); after copy_blocks and the scatter of the child's
    new token, the child's paged attention equals plain float64 attention
    (torch SDPA) over the parent's tokens followed by the child's token, and
    the parent's own attention is unchanged.
  * The copy moves whole blocks (every head, every slot) and touches nothing
    else: checked through a flat slot view of the pools.
  * Calls that would make the result depend on the order of the copies are
    rejected.
"""

import math

import numpy as np
import pytest
import torch

from oracle import allocator as al
from oracle import attention as att
from oracle import copy as cp
from oracle import scatter as sc


def _sdpa(q, k, v):
    """float64 attention of q [Hq, D] over k, v [Hkv, T, D] (GQA by repeat)."""
    G = q.shape[0] // k.shape[0]
    qt = torch.from_numpy(q)[:, None, :]
    kt = torch.from_numpy(k).repeat_interleave(G, dim=0)
    vt = torch.from_numpy(v).repeat_interleave(G, dim=0)
    return torch.nn.functional.scaled_dot_product_attention(qt[None], kt[None], vt[None])[0, :, 0, :].numpy()


def cow_end_to_end_holds(parent_len, copy_fn=cp.copy_blocks):
    """True when the child's and the parent's paged attention after the
    copy-on-write equal plain attention over their token sequences."""
    rng = np.random.default_rng(parent_len)
    bs, nb, h_kv, h_q, d = 4, 24, 2, 4, 8
    bm = al.BlockManager(nb, bs, free_order=rng.permutation(nb))
    kc = rng.standard_normal((nb, h_kv, bs, d)).astype(np.float32)
    vc = rng.standard_normal((nb, h_kv, bs, d)).astype(np.float32)
    # the parent's tokens, written in order through the allocator's slots
    toks_k = rng.standard_normal((parent_len, h_kv, d)).astype(np.float32)
    toks_v = rng.standard_normal((parent_len, h_kv, d)).astype(np.float32)
    slots, _ = bm.append(0, parent_len)
    kc, vc = sc.reshape_and_cache(toks_k.view(np.uint32), toks_v.view(np.uint32), kc.view(np.uint32),
                                  vc.view(np.uint32), slots, in_dtype="f32", kv_dtype="f32", block_size=bs)
    bm.fork(0, 1)
    new_slots, (src, dst) = bm.append(1, 1)
    partial = parent_len % bs != 0
    assert (src >= 0) == partial
    if partial:
        kc, vc = copy_fn(kc, vc, [[src, dst]])
    new_k = rng.standard_normal((1, h_kv, d)).astype(np.float32)
    new_v = rng.standard_normal((1, h_kv, d)).astype(np.float32)
    kc, vc = sc.reshape_and_cache(new_k.view(np.uint32), new_v.view(np.uint32), kc, vc, new_slots,
                                  in_dtype="f32", kv_dtype="f32", block_size=bs)
    q = rng.standard_normal((2, h_q, d)).astype(np.float32)
    mb = max(len(bm.block_table(s)[0]) for s in (0, 1))
    bt = np.full((2, mb), -1, dtype=np.int32)
    lens = np.zeros(2, dtype=np.int32)
    for s in (0, 1):
        table, n = bm.block_table(s)
        bt[s, :len(table)] = table
        lens[s] = n
    out = att.paged_attention_decode(q.view(np.uint32), kc, vc, bt, lens, q_dtype="f32", kv_dtype="f32", block_size=bs)
    k_all = np.concatenate([toks_k, new_k]).transpose(1, 0, 2).astype(np.float64)
    v_all = np.concatenate([toks_v, new_v]).transpose(1, 0, 2).astype(np.float64)
    child_ok = np.allclose(out[1], _sdpa(q[1].astype(np.float64), k_all, v_all), rtol=1e-12, atol=1e-12)
    parent_ok = np.allclose(out[0], _sdpa(q[0].astype(np.float64), k_all[:, :parent_len], v_all[:, :parent_len]),
                            rtol=1e-12, atol=1e-12)
    return bool(child_ok and parent_ok)


@pytest.mark.parametrize("parent_len", [5, 13, 19, 8])
def test_copy_on_write_end_to_end(parent_len):
    assert cow_end_to_end_holds(parent_len)


def _k_only(kc, vc, pairs):
    k, _ = cp.copy_blocks(kc, vc, pairs)
    return k, np.array(vc, copy=True)


def _first_head_only(kc, vc, pairs):
    k, v = np.array(kc, copy=True), np.array(vc, copy=True)
    for src, dst in pairs:
        k[dst, 0], v[dst, 0] = kc[src, 0], vc[src, 0]
    return k, v


def _swapped(kc, vc, pairs):
    return cp.copy_blocks(kc, vc, [[d, s] for s, d in pairs])


@pytest.mark.parametrize("mutant", [_k_only, _first_head_only, _swapped], ids=lambda f: f.__name__)
def test_planted_copy_mistake_is_caught(mutant):
    assert not all(cow_end_to_end_holds(n, mutant) for n in (5, 13, 19))


def test_copy_moves_whole_blocks_and_nothing_else():
    rng = np.random.default_rng(3)
    nb, h_kv, bs, d = 10, 3, 4, 5
    kc = rng.integers(0, 2 ** 16, (nb, h_kv, bs, d)).astype(np.uint16)
    vc = rng.integers(0, 2 ** 16, (nb, h_kv, bs, d)).astype(np.uint16)
    pairs = [[2, 7], [5, 0], [9, 3]]
    ko, vo = cp.copy_blocks(kc, vc, pairs)
    flat = lambda c: np.transpose(c, (0, 2, 1, 3)).reshape(nb * bs, h_kv, d)  # slot-major view
    fk, fv, fko, fvo = flat(kc), flat(vc), flat(ko), flat(vo)
    moved = {dst: src for src, dst in pairs}
    for slot in range(nb * bs):
        b, o = divmod(slot, bs)
        src_slot = moved[b] * bs + o if b in moved else slot
        assert np.array_equal(fko[slot], fk[src_slot]) and np.array_equal(fvo[slot], fv[src_slot])


@pytest.mark.parametrize("pairs", [[[1, 2], [3, 2]], [[1, 2], [2, 3]], [[0, 10]], [[-1, 2]]])
def test_order_dependent_or_out_of_range_calls_rejected(pairs):
    kc = np.zeros((10, 1, 2, 2), np.float32)
    with pytest.raises(ValueError):
        cp.copy_blocks(kc, kc, pairs)
