"""copy_blocks: the block copy that completes copy-on-write; swap_blocks: the
block move between a device pool and a host pool that preemption by swapping
makes.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sequences share prefix blocks by reference; when a sequence appends into a
shared block that is only partly filled, it moves onto a fresh block first
([OT] "Block Tables and Sharing"; [AF] "The bonus: sharing via
copy-on-write").  The block manager reports that move as a (src, dst) pair;
this step copies the whole physical block src (every KV head, every slot) to
dst, in the K pool and in the V pool, so that the sequence's existing tokens
are intact in its new block before the new token is written.

Reading taken here: all pairs of one call are applied to the pools as they
were before the call; a block may not be both a source and a destination in
one call, and no destination may repeat (those calls are rejected).
"""

import numpy as np


def copy_blocks(k_cache, v_cache, pairs):
    """Return (k_cache, v_cache) copies with block dst := block src for every
    (src, dst) row of pairs ([n, 2] int)."""
    pairs = np.asarray(pairs, dtype=np.int64).reshape(-1, 2)
    num_blocks = k_cache.shape[0]
    srcs, dsts = pairs[:, 0].tolist(), pairs[:, 1].tolist()
    if len(set(dsts)) != len(dsts):
        raise ValueError("a destination block repeats")
    if set(srcs) & set(dsts):
        raise ValueError("a block is both a source and a destination")
    for b in srcs + dsts:
        if not 0 <= b < num_blocks:
            raise ValueError(f"block id {b} outside a pool of {num_blocks} blocks")
    k_out = np.array(k_cache, copy=True)
    v_out = np.array(v_cache, copy=True)
    for src, dst in zip(srcs, dsts):
        k_out[dst] = k_cache[src]
        v_out[dst] = v_cache[src]
    return k_out, v_out


# ---------------------------------------------------------------- swapping
#
# When the device pool fills, a running sequence can be preempted by moving
# its KV blocks to host memory and paging them back later instead of
# recomputing them ([AF] "Beyond paging: radix trees and continuous
# batching"; [OT] "Offload").  The move itself is a block copy between two
# different pools; the sequence comes back into whatever device blocks the
# allocator hands out then, with a new block table.
#
# Readings: block s of the source pools goes to block d of the destination
# pools, every KV head and slot, K and V; a destination may not repeat and
# every id must lie inside its pool (those calls are rejected).


def swap_blocks(dst_k, dst_v, src_k, src_v, pairs):
    """Return (dst_k, dst_v) copies with block d := block s of (src_k, src_v)
    for every (s, d) row of pairs ([n, 2] int)."""
    pairs = np.asarray(pairs, dtype=np.int64).reshape(-1, 2)
    if dst_k.shape[1:] != src_k.shape[1:] or dst_v.shape != dst_k.shape or src_v.shape != src_k.shape:
        raise ValueError("pools disagree in [h_kv, block_size, head_dim]")
    srcs, dsts = pairs[:, 0].tolist(), pairs[:, 1].tolist()
    if len(set(dsts)) != len(dsts):
        raise ValueError("a destination block repeats")
    for b in srcs:
        if not 0 <= b < src_k.shape[0]:
            raise ValueError(f"source block {b} outside a pool of {src_k.shape[0]} blocks")
    for b in dsts:
        if not 0 <= b < dst_k.shape[0]:
            raise ValueError(f"destination block {b} outside a pool of {dst_k.shape[0]} blocks")
    k_out = np.array(dst_k, copy=True)
    v_out = np.array(dst_v, copy=True)
    for s, d in zip(srcs, dsts):
        k_out[d] = src_k[s]
        v_out[d] = src_v[s]
    return k_out, v_out
