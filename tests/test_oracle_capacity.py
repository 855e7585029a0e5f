"""Pins of oracle.capacity against the values the pages print.

Every expected number comes from tests/golden/pages_capacity.txt, where each
line names the page and section that prints it.
"""

import pytest

from oracle import capacity as cap

GIB12 = 12 * 2 ** 30


def test_bytes_per_token(pages_capacity):
    assert cap.kv_bytes_per_token(80, 8, 128, 2) == pages_capacity["gqa_bf16_bytes_per_token"]
    assert cap.kv_bytes_per_token(80, 64, 128, 2) == pages_capacity["mha64_bf16_bytes_per_token"]
    assert cap.kv_bytes_per_token(80, 8, 128, 1) == pages_capacity["gqa_fp8_bytes_per_token"]
    # 8x footprint gap of 64-head MHA vs 8-KV-head GQA
    assert cap.kv_bytes_per_token(80, 64, 128, 2) == 8 * cap.kv_bytes_per_token(80, 8, 128, 2)


def test_twelve_gib_pool(pages_capacity):
    bpt = cap.kv_bytes_per_token(80, 8, 128, 2)
    assert GIB12 == pages_capacity["budget_bytes"]
    pool = cap.carve(GIB12, bpt, 16)
    assert pool.token_slots == pages_capacity["token_slots_12gib"]
    assert pool.blocks == pages_capacity["pool_blocks_12gib_b16"]
    assert pool.block_slots == pages_capacity["block_backed_slots_12gib_b16"]
    assert pool.leftover_bytes == pages_capacity["leftover_bytes_12gib_b16"]
    assert round(pool.leftover_bytes / bpt, 1) == 9.6


def test_825_token_request(pages_capacity):
    r = cap.footprint(825, 16, reserved_tokens=2048)
    assert r.blocks == pages_capacity["request_825_blocks_b16"]
    assert r.slots == pages_capacity["request_825_slots_b16"]
    assert r.unused_slots == pages_capacity["request_825_unused_b16"]
    assert round(100 * r.waste_fraction, 4) == pages_capacity["request_825_waste_percent_b16"]
    assert round(2048 / r.slots, 4) == pages_capacity["request_825_allocation_ratio"]
    assert 2048 - 825 == pages_capacity["request_825_contiguous_unused"]
    assert round(100 * (2048 - 825) / 2048, 2) == pages_capacity["request_825_contiguous_unused_percent"]


def test_request_capacity(pages_capacity):
    bpt = cap.kv_bytes_per_token(80, 8, 128, 2)
    pool = cap.carve(GIB12, bpt, 16)
    contiguous = cap.contiguous_admissions(pool.token_slots, 2048)
    paged = cap.paged_admissions(pool.blocks, 16, 825)
    assert contiguous == pages_capacity["contiguous_requests_825_of_2048"]
    assert paged == pages_capacity["paged_requests_825"]
    assert round(paged / contiguous, 4) == pages_capacity["capacity_ratio_825"]
    need48 = 48 * cap.footprint(825, 16).slots
    assert need48 == pages_capacity["slots_for_48_requests_825"]
    assert need48 > pool.block_slots  # the 48th request does not fit


def test_fp8_and_broken_cases(pages_capacity):
    fp8 = cap.carve(GIB12, cap.kv_bytes_per_token(80, 8, 128, 1), 16)
    assert fp8.token_slots == pages_capacity["token_slots_12gib_fp8"]
    assert cap.footprint(825, 32).blocks == pages_capacity["request_825_blocks_b32"]
    assert cap.footprint(825, 32).slots == cap.footprint(825, 16).slots
    assert cap.footprint(200, 16).slots == pages_capacity["request_200_slots_b16"]
    assert cap.footprint(200, 32).slots == pages_capacity["request_200_slots_b32"]
    wrong = cap.carve(GIB12, cap.kv_bytes_per_token(80, 64, 128, 2), 16)
    assert wrong.token_slots == pages_capacity["token_slots_12gib_64_heads"]
    # a 4-5x allocation ratio is not what this workload gives
    assert not 4.0 <= 2048 / cap.footprint(825, 16).slots <= 5.0


def test_prefix_granularity(pages_capacity):
    # block-granular matching reuses only whole blocks of the prompt
    whole = (103 // 16) * 16
    assert whole == pages_capacity["prefix_103_reusable_b16"]


def test_other_pages_examples(pages_capacity):
    dense = cap.kv_bytes_per_token(32, 32, 128, 2)
    assert dense == pages_capacity["dense8b_f16_bytes_per_token"]
    assert 4096 * dense == pages_capacity["dense8b_f16_bytes_4096_tokens"]
    gqa = cap.kv_bytes_per_token(80, 8, 128, 2)
    approx = pages_capacity["approx_70b_gqa_bytes_per_token"]
    assert abs(gqa - approx) / approx < 0.10
    approx8k = pages_capacity["approx_70b_gqa_bytes_8000_tokens"]
    assert abs(8000 * gqa - approx8k) / approx8k < 0.10
    # the 8B GQA preset against the 7B model without GQA ([UD] "The maths"):
    # 8 against 32 KV heads, a quarter of the bytes
    assert cap.kv_bytes_per_token(32, 8, 128, 2) * 4 == cap.kv_bytes_per_token(32, 32, 128, 2)


@pytest.mark.parametrize("tokens,block,reserved", [(0, 16, 2048), (-5, 16, 2048), (10, 0, 2048), (3000, 16, 2048)])
def test_invalid_inputs_rejected(tokens, block, reserved):
    with pytest.raises(ValueError):
        cap.footprint(tokens, block, reserved_tokens=reserved)


def test_tail_waste_bound_exhaustive():
    # only the final block can be partly empty: waste <= block_size - 1
    for bs in (1, 2, 3, 16, 32):
        for n in range(1, 400):
            r = cap.footprint(n, bs)
            assert 0 <= r.unused_slots <= bs - 1
            assert r.slots - bs < n <= r.slots
