"""Paged decode attention, written as its plain definition.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix
  * Each sequence's KV cache is cut into fixed-size blocks stored anywhere in
    the pool; a per-sequence block table maps logical block j to a physical
    block ([UD] intro; [AF] "PagedAttention: virtual memory for GPUs").
  * To the model the tokens remain one unbroken sequence; only the
    addressing changes, the attention kernel following the block table
    rather than reading a contiguous copy ([OT] "Block Tables and Sharing";
    [AF] "PagedAttention").
  * Decoding attends the new token's query over the cached K/V of the tokens
    already processed ([AF] "What the KV cache actually is").

So paging changes only the addressing, and the exact result is textbook
scaled-dot-product attention over the logical sequence.  This module computes
exactly that: step 1 turns each block table back into a contiguous K/V (the
gather the kernel avoids), step 2 is softmax(q K^T * scale) V in float64.

Readings of what the pages leave open (each one stated where it is used):
  * scale defaults to 1/sqrt(head_dim) and the caller may override it;
  * grouped-query attention: query head g reads KV head g // (h_q / h_kv)
    (contiguous groups; [OT] "Reproduce Bytes per Token" and [UD] "The maths"
    only say that query heads share KV heads);
  * positions t >= context_len (the unused tail of the last block, [OT]
    "Internal Fragmentation") and block-table entries past the last used block
    are never read, whatever they hold;
  * a sequence with context_len 0 attends over nothing: its output is 0;
  * FP8 pools: a stored code c stands for decode(c) * scale (codecs.py).

Layouts (row-major, as the GPU path receives them)
  q            [num_seqs, h_q, head_dim]               stored bits
  k_cache      [num_blocks, h_kv, block_size, head_dim] stored bits
  v_cache      same as k_cache
  block_tables [num_seqs, max_blocks_per_seq] int32
  context_lens [num_seqs] int32
"""

import math

import numpy as np

from .codecs import bits_to_f64


def kv_head_of(q_head: int, h_q: int, h_kv: int) -> int:
    """KV head read by a query head: contiguous groups of h_q / h_kv heads."""
    group = h_q // h_kv
    return q_head // group


def resolve_sequence(cache_bits, block_row, context_len, block_size, dtype, scale=1.0):
    """Contiguous float64 K (or V) of one sequence: [h_kv, context_len, head_dim].

    Logical position t lives in physical block block_row[t // block_size] at
    offset t % block_size.  Only positions t < context_len are touched.
    """
    h_kv, head_dim = cache_bits.shape[1], cache_bits.shape[3]
    out = np.empty((h_kv, context_len, head_dim), dtype=np.float64)
    num_logical = -(-context_len // block_size)
    for j in range(num_logical):
        phys = int(block_row[j])
        if not 0 <= phys < cache_bits.shape[0]:
            raise ValueError(f"block id {phys} out of range for logical block {j}")
        first = j * block_size
        used = min(block_size, context_len - first)  # tail slots are never read
        out[:, first:first + used, :] = bits_to_f64(cache_bits[phys, :, :used, :], dtype) * scale
    return out


def attend(q_vec, keys, values, scale):
    """softmax(scale * keys @ q) @ values for one query row, in float64."""
    n = keys.shape[0]
    if n == 0:
        return np.zeros(values.shape[1], dtype=np.float64)
    logits = scale * (keys @ q_vec)
    peak = np.max(logits)
    weights = np.exp(logits - peak)
    return (weights @ values) / np.sum(weights)


def paged_attention_decode(q, k_cache, v_cache, block_tables, context_lens, *,
                           q_dtype, kv_dtype, block_size, scale=None,
                           k_scale=1.0, v_scale=1.0, seqs=None, heads=None):
    """Float64 output [num_seqs, h_q, head_dim] of paged decode attention.

    seqs / heads: optional subsets of sequence and query-head indices to
    compute (the rest of the returned array is NaN); lets tests sample very
    large workloads one output row at a time.
    """
    num_seqs, h_q, head_dim = q.shape
    h_kv = k_cache.shape[1]
    if h_q % h_kv != 0:
        raise ValueError("h_q must be a multiple of h_kv")
    if k_cache.shape[2] != block_size:
        raise ValueError("k_cache block dimension must equal block_size")
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    max_blocks = block_tables.shape[1]
    out = np.full((num_seqs, h_q, head_dim), np.nan, dtype=np.float64)
    seq_list = range(num_seqs) if seqs is None else seqs
    for s in seq_list:
        ctx = int(context_lens[s])
        if not 0 <= ctx <= max_blocks * block_size:
            raise ValueError(f"context length {ctx} of sequence {s} out of range")
        keys = resolve_sequence(k_cache, block_tables[s], ctx, block_size, kv_dtype, k_scale)
        vals = resolve_sequence(v_cache, block_tables[s], ctx, block_size, kv_dtype, v_scale)
        q_s = bits_to_f64(q[s], q_dtype)
        head_list = range(h_q) if heads is None else heads
        for g in head_list:
            kvh = kv_head_of(g, h_q, h_kv)
            out[s, g] = attend(q_s[g], keys[kvh], vals[kvh], scale)
    return out


# ---------------------------------------------------------------- several new query tokens
#
# What the pages fix
#   * every token already processed keeps its K and V so that the tokens after
#     it can attend to them ([UD] intro): attention runs forward in position,
#     a token sees the positions before it;
#   * a prompt whose prefix is already cached recomputes only its trailing
#     tokens over that prefix ([AF] "Beyond paging: radix trees and continuous
#     batching"), and speculative decoding adds lookahead tokens past the
#     committed ones ([OT] "Internal Fragmentation"): one step can bring
#     several new tokens of one sequence.
# Readings of what the pages leave open
#   * the m new tokens of a sequence are the last m of its context_len cached
#     tokens (their K/V already written), so new token i sits at position
#     context_len - m + i;
#   * a token attends to its own position too (its K/V are cached like the
#     others) and to no later one;
#   * a token with no position to attend to (more new tokens than cached
#     ones) gets 0, as an empty context does for decode.


def causal_visible(context_len: int, num_new: int, i: int) -> int:
    """How many positions new token i (of num_new) attends to: [0, ctx - m + i]."""
    return max(0, context_len - num_new + i + 1)


def paged_attention_multi(q, k_cache, v_cache, block_tables, context_lens, query_start, *,
                          q_dtype, kv_dtype, block_size, scale=None, k_scale=1.0, v_scale=1.0, seqs=None):
    """Float64 output [num_query_tokens, h_q, head_dim] for several new tokens per sequence.

    q: [T, h_q, head_dim] stored bits; rows query_start[s] .. query_start[s+1]-1
    are the new tokens of sequence s in order.  Rows of sequences not in
    `seqs` (and rows no sequence owns) are NaN.
    """
    T, h_q, head_dim = q.shape
    num_seqs = len(context_lens)
    h_kv = k_cache.shape[1]
    if h_q % h_kv != 0:
        raise ValueError("h_q must be a multiple of h_kv")
    if k_cache.shape[2] != block_size:
        raise ValueError("k_cache block dimension must equal block_size")
    if len(query_start) != num_seqs + 1:
        raise ValueError("query_start needs num_seqs + 1 entries")
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    max_blocks = block_tables.shape[1]
    out = np.full((T, h_q, head_dim), np.nan, dtype=np.float64)
    for s in (range(num_seqs) if seqs is None else seqs):
        q0, q1 = int(query_start[s]), int(query_start[s + 1])
        if not 0 <= q0 <= q1 <= T:
            raise ValueError(f"query rows [{q0}, {q1}) of sequence {s} out of range")
        m = q1 - q0
        ctx = int(context_lens[s])
        if not 0 <= ctx <= max_blocks * block_size:
            raise ValueError(f"context length {ctx} of sequence {s} out of range")
        keys = resolve_sequence(k_cache, block_tables[s], ctx, block_size, kv_dtype, k_scale)
        vals = resolve_sequence(v_cache, block_tables[s], ctx, block_size, kv_dtype, v_scale)
        for i in range(m):
            n = causal_visible(ctx, m, i)
            q_i = bits_to_f64(q[q0 + i], q_dtype)
            for g in range(h_q):
                kvh = kv_head_of(g, h_q, h_kv)
                out[q0 + i, g] = attend(q_i[g], keys[kvh, :n], vals[kvh, :n], scale)
    return out
