"""copy_blocks: the block copy that completes copy-on-write.

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
