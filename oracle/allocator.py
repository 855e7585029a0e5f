"""Block manager: on-demand allocation, free list, refcounts, copy-on-write.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix
  * Blocks are handed out only as a sequence actually grows ([UD] intro;
    [AF] "PagedAttention": new blocks are allocated on demand).
  * A sequence that grows takes free blocks one by one, as it needs them;
    the blocks it already holds stay where they are ([OT] "Answer Key",
    question 2).
  * A physical block goes back to the free list once no sequence references
    it ([OT] "Block Tables and Sharing").
  * Reference counting lets sequences point at the same prefix blocks; a
    fresh block is allocated only when two sequences diverge inside a shared
    tail block ([OT] "Block Tables and Sharing"; [AF] "The bonus: sharing via
    copy-on-write").
  * Only the final block of a sequence can be partly empty, so tail waste is
    at most block_size - 1 slots ([OT] "Internal Fragmentation").
  * Admission can fail when the pool has no room ([OT] "Worked Capacity Under a
    12 GiB KV Budget": a 48th 825-token request does not fit).

Readings of what the pages leave open
  * The free list is FIFO: blocks are taken from the front; a block whose
    refcount reaches zero is appended at the back; a freed sequence releases
    its blocks in block-table order.  The initial order is the caller's.
  * A sequence's next token needs a new block exactly when its length is a
    multiple of block_size.
  * Appending to a sequence whose last block is partly filled and shared
    (refcount > 1) first moves the sequence onto a fresh block (copy-on-write):
    the call reports (src, dst) so that the caller can copy the filled slots,
    and the old block loses one reference.
  * An append that cannot get every block it needs changes nothing.
"""

from collections import deque


class OutOfBlocks(Exception):
    """The pool cannot supply the blocks an append needs (nothing changed)."""


class InvalidRequest(Exception):
    """Bad argument: unknown or duplicate sequence, negative count, ..."""


class BlockManager:
    def __init__(self, num_blocks, block_size, free_order=None):
        if num_blocks <= 0 or block_size <= 0:
            raise InvalidRequest("num_blocks and block_size must be positive")
        order = list(range(num_blocks)) if free_order is None else [int(b) for b in free_order]
        if sorted(order) != list(range(num_blocks)):
            raise InvalidRequest("free_order must be a permutation of the pool")
        self.block_size = block_size
        self.num_blocks = num_blocks
        self.free = deque(order)
        self.refcount = [0] * num_blocks
        self.tables = {}   # seq -> list of physical block ids
        self.lengths = {}  # seq -> tokens held

    def append(self, seq, n_tokens):
        """Give `seq` n_tokens more token slots; return (slots, (cow_src, cow_dst))."""
        if seq < 0 or n_tokens < 0:
            raise InvalidRequest("sequence id and token count must be non-negative")
        table = self.tables.get(seq, [])
        length = self.lengths.get(seq, 0)
        bs = self.block_size
        cow = n_tokens > 0 and length % bs != 0 and self.refcount[table[-1]] > 1
        blocks_after = -(-(length + n_tokens) // bs)
        needed = (blocks_after - len(table)) + (1 if cow else 0)
        if needed > len(self.free):
            raise OutOfBlocks(f"need {needed} blocks, {len(self.free)} free")
        table = list(table)
        cow_pair = (-1, -1)
        if cow:
            src = table[-1]
            dst = self.free.popleft()
            self.refcount[src] -= 1
            self.refcount[dst] = 1
            table[-1] = dst
            cow_pair = (src, dst)
        slots = []
        for _ in range(n_tokens):
            if length % bs == 0:
                fresh = self.free.popleft()
                self.refcount[fresh] = 1
                table.append(fresh)
            slots.append(table[length // bs] * bs + length % bs)
            length += 1
        self.tables[seq] = table
        self.lengths[seq] = length
        return slots, cow_pair

    def fork(self, parent, child):
        """`child` starts as a copy of `parent` that shares all its blocks."""
        if parent not in self.tables or child in self.tables or child < 0:
            raise InvalidRequest("fork needs an existing parent and a new child id")
        self.tables[child] = list(self.tables[parent])
        self.lengths[child] = self.lengths[parent]
        for b in self.tables[child]:
            self.refcount[b] += 1

    def free_seq(self, seq):
        """Drop `seq`; blocks nobody references any more return to the free list."""
        if seq not in self.tables:
            raise InvalidRequest("unknown sequence")
        for b in self.tables.pop(seq):
            self.refcount[b] -= 1
            if self.refcount[b] == 0:
                self.free.append(b)
        del self.lengths[seq]

    def block_table(self, seq):
        if seq not in self.tables:
            raise InvalidRequest("unknown sequence")
        return list(self.tables[seq]), self.lengths[seq]

    def num_free(self):
        return len(self.free)
