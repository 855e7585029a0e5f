"""Sizing arithmetic of a paged KV pool.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The headline bandwidth figures are priced in KV bytes per token, so that
count, and the way a byte budget turns into tokens and blocks, are checked
here against every value the pages print (tests/golden/pages_capacity.txt).

Definitions used ([OT] = the "Paged KV Cache" tutorial, [UD] = "AI
Engineering Visualised: KV cache", [AF] = "KV cache and PagedAttention in
serving"):
  * One token's KV state is a K row and a V row of head_dim elements for each
    KV head of each layer ([OT] "Reproduce Bytes per Token"; [UD] "The
    maths"; [AF] "What the KV cache actually is" counts attention heads,
    which coincide with KV heads only without grouped-query attention).
  * A byte budget holds as many whole token slots as fit, and as many whole
    blocks of block_size slots as fit; what is left over cannot hold a block
    ([OT] "Worked Capacity Under a 12 GiB KV Budget").
  * Under paging a request's footprint is what the block manager hands it:
    this module grows the request in the oracle's own block manager
    (allocator.py, blocks claimed on demand) and reads its table, rather
    than restating a formula ([OT] "Worked Example: The 825-Token Request",
    "Internal Fragmentation").
  * A contiguous reservation sets aside the declared maximum length for each
    request ([OT] "Reservation Waste"; [UD] "The maths").
  * Lengths and block sizes below one token are rejected ([OT] "Build the
    Capacity Calculator").
"""

from dataclasses import dataclass

from .allocator import BlockManager, OutOfBlocks


def kv_bytes_per_token(layers, kv_heads, head_dim, bytes_per_element):
    """KV bytes one token adds: K and V rows for every (layer, KV head)."""
    dims = (layers, kv_heads, head_dim, bytes_per_element)
    if min(dims) < 1:
        raise ValueError(f"model dimensions must all be at least 1, got {dims}")
    rows_per_token = 2 * layers * kv_heads  # one K and one V row per layer and KV head
    return rows_per_token * head_dim * bytes_per_element


@dataclass(frozen=True)
class Pool:
    """How a byte budget divides into token slots and blocks."""
    token_slots: int     # whole tokens of KV state the budget holds
    blocks: int          # whole blocks of block_size token slots
    block_slots: int     # token slots those blocks provide
    leftover_bytes: int  # bytes short of one more whole block


def carve(budget_bytes, bytes_per_token, block_size):
    if block_size < 1:
        raise ValueError(f"a block holds at least one token, got block_size={block_size}")
    block_bytes = bytes_per_token * block_size
    blocks, leftover = divmod(budget_bytes, block_bytes)
    return Pool(budget_bytes // bytes_per_token, blocks, blocks * block_size, leftover)


@dataclass(frozen=True)
class Footprint:
    """What one request occupies under paging."""
    tokens: int
    blocks: int
    slots: int

    @property
    def unused_slots(self):
        return self.slots - self.tokens

    @property
    def waste_fraction(self):
        return self.unused_slots / self.slots


def footprint(tokens, block_size, reserved_tokens=None):
    """Grow one request of `tokens` tokens in a block manager whose pool can
    hold it, and read back the blocks it was handed."""
    if block_size < 1:
        raise ValueError(f"a block holds at least one token, got block_size={block_size}")
    if tokens < 1:
        raise ValueError(f"a request holds at least one token, got {tokens}")
    if reserved_tokens is not None and tokens > reserved_tokens:
        raise ValueError(f"a {tokens}-token request outgrows its {reserved_tokens}-token reservation")
    manager = BlockManager(tokens + 1, block_size)  # never the limit: a block holds >= 1 token
    manager.append(0, tokens)
    table, held = manager.block_table(0)
    assert held == tokens
    return Footprint(tokens, len(table), len(table) * block_size)


def contiguous_admissions(token_slots, reserved_tokens):
    """Requests a pool of token_slots admits when each reserves
    reserved_tokens contiguous slots up front."""
    return token_slots // reserved_tokens


def paged_admissions(num_blocks, block_size, tokens):
    """Requests of `tokens` tokens a pool of num_blocks blocks admits under
    paging: admit one after another into the oracle's block manager until
    an append is refused."""
    manager = BlockManager(num_blocks, block_size)
    admitted = 0
    while True:
        try:
            manager.append(admitted, tokens)
        except OutOfBlocks:
            return admitted
        admitted += 1
