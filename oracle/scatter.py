"""reshape_and_cache: write each new token's K/V into its slot of the block pool.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Per the pages, a growing sequence takes free blocks one by one and its
earlier blocks never move ([OT] "Answer Key", question 2), and a block table
maps each logical position to a physical block ([UD] intro).  The step
that puts a freshly computed token into that pool is not spelled out there;
the reading taken here is the plainest one: a token's slot is

    slot = physical_block * block_size + offset_in_block

and its K (and V) vector for every KV head lands at
k_cache[slot // block_size, head, slot % block_size, :].  A negative slot
marks a padding token that is not written.  Two tokens with one slot in the
same call are a caller error (which write wins is not defined).

Element conversion
  * same storage type in and out: the bits are copied unchanged;
  * into an FP8 pool: binary32 value -> one correctly-rounded binary32
    division by the tensor's scale -> nearest E4M3 code (codecs.py).
"""

import numpy as np

from .codecs import bits_to_f64, quantize_e4m3


def reshape_and_cache(key, value, k_cache, v_cache, slot_mapping, *, in_dtype,
                      kv_dtype, block_size, k_scale=1.0, v_scale=1.0):
    """Return (k_cache, v_cache) copies with the new tokens written in.

    key, value   [num_tokens, h_kv, head_dim] stored bits of in_dtype
    k_cache ...  [num_blocks, h_kv, block_size, head_dim] stored bits
    slot_mapping [num_tokens] int64
    """
    k_out = np.array(k_cache, copy=True)
    v_out = np.array(v_cache, copy=True)
    num_blocks = k_cache.shape[0]
    for i, slot in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
        slot = int(slot)
        if slot < 0:
            continue
        block, offset = divmod(slot, block_size)
        if block >= num_blocks:
            raise ValueError(f"slot {slot} outside a pool of {num_blocks} blocks")
        k_out[block, :, offset, :] = _encode(key[i], in_dtype, kv_dtype, k_scale)
        v_out[block, :, offset, :] = _encode(value[i], in_dtype, kv_dtype, v_scale)
    return k_out, v_out


def _encode(bits, in_dtype, kv_dtype, scale):
    if in_dtype == kv_dtype:
        return bits
    if kv_dtype == "fp8":
        # Every f32 / f16 / bf16 value is exact in binary32, so widening first
        # loses nothing; the only rounding is the division and the E4M3 step.
        as_f32 = bits_to_f64(bits, in_dtype).astype(np.float32)
        return quantize_e4m3(as_f32, scale)
    raise ValueError(f"no conversion from {in_dtype} to {kv_dtype}")
