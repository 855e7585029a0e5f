"""Sizing arithmetic of a paged KV pool, restated from the pages.

TEST INFRASTRUCTURE ONLY (see the package docstring).

This is the exact integer arithmetic the pages walk through; it fixes the
per-token byte count that the bandwidth figures are priced with, and it is
checked against every value the pages print (tests/golden/pages_capacity.txt).

  * Per-token KV state: K and V, at every layer, for every KV head, head_dim
    elements of bytes_per_element each ([OT] "Reproduce Bytes per Token";
    [UD] "The maths"; [AF] "What the KV cache actually is" writes "heads",
    which is right only without grouped-query attention).
  * Whole token slots in a byte budget, and whole blocks of block_size slots
    ([OT] "Worked Capacity Under a 12 GiB KV Budget").
  * A request of n tokens takes ceil(n / block_size) blocks; only the final
    block can be partly empty ([OT] "Worked Example: The 825-Token Request",
    "Internal Fragmentation"; [UD] "The maths", paged waste).
  * Contiguous reservation holds the declared maximum for every request
    ([OT] "Reservation Waste"; [UD] "The maths", contiguous waste).
  * Invalid lengths or block sizes are rejected ([OT] "Build the Capacity
    Calculator").
"""

from dataclasses import dataclass


def kv_bytes_per_token(layers, kv_heads, head_dim, bytes_per_element):
    """Two tensors (K and V) x layers x KV heads x head_dim x element bytes."""
    for v in (layers, kv_heads, head_dim, bytes_per_element):
        if v <= 0:
            raise ValueError("model dimensions must be positive")
    return 2 * layers * kv_heads * head_dim * bytes_per_element


def token_slots(budget_bytes, bytes_per_token):
    """Whole tokens of KV state that fit in the budget."""
    return budget_bytes // bytes_per_token


def pool_blocks(budget_bytes, bytes_per_token, block_size):
    """Whole blocks of block_size tokens that fit in the budget."""
    if block_size <= 0:
        raise ValueError("block size must be positive")
    return budget_bytes // (bytes_per_token * block_size)


def blocks_for(tokens, block_size):
    """Blocks a sequence of `tokens` tokens occupies: ceil(tokens / block_size)."""
    if block_size <= 0 or tokens < 0:
        raise ValueError("invalid sequence or block size")
    return -(-tokens // block_size)


@dataclass(frozen=True)
class PagedRequest:
    tokens: int
    blocks: int
    slots: int
    unused_slots: int
    waste_fraction: float


def paged_request(tokens, block_size, reserved_tokens=None):
    """Footprint of one request under paging (and a check against its reservation)."""
    if tokens <= 0 or block_size <= 0:
        raise ValueError("invalid sequence or block size")
    if reserved_tokens is not None and tokens > reserved_tokens:
        raise ValueError("invalid sequence or block size")
    blocks = blocks_for(tokens, block_size)
    slots = blocks * block_size
    return PagedRequest(tokens, blocks, slots, slots - tokens, (slots - tokens) / slots)


def contiguous_requests(slots, reserved_tokens):
    """Requests that fit when each one reserves reserved_tokens contiguous slots."""
    return slots // reserved_tokens


def paged_requests(num_pool_blocks, blocks_per_request):
    """Requests that fit when each one holds blocks_per_request whole blocks."""
    return num_pool_blocks // blocks_per_request


def leftover_bytes(budget_bytes, bytes_per_token, block_size):
    """Budget bytes too few to form one more whole block."""
    return budget_bytes - pool_blocks(budget_bytes, bytes_per_token, block_size) * block_size * bytes_per_token
