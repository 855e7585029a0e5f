"""Pins of oracle.codecs: closed forms of the formats, exhaustive code checks,
and cross-checks against PyTorch's own dtype conversions (a library routine the
oracle does not use)."""

import numpy as np
import pytest
import torch

from oracle import codecs


def torch_e4m3_decode(codes):
    return torch.from_numpy(codes.astype(np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_e4m3_all_codes_match_library():
    codes = np.arange(256, dtype=np.uint8)
    ours = codecs.e4m3_to_f64(codes)
    ref = torch_e4m3_decode(codes)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    assert np.array_equal(np.signbit(ours[ok]), np.signbit(ref[ok]))


def test_e4m3_closed_forms():
    val = lambda c: float(codecs.e4m3_to_f64(np.array([c], np.uint8))[0])
    assert val(0x7E) == 448.0                 # largest finite: 1.75 * 2^8
    assert val(0xFE) == -448.0
    assert val(0x01) == 2.0 ** -9             # smallest subnormal: 1/8 * 2^-6
    assert val(0x07) == 7 * 2.0 ** -9         # largest subnormal
    assert val(0x08) == 2.0 ** -6             # smallest normal
    assert val(0x38) == 1.0                   # exponent field 7 == bias
    assert val(0x00) == 0.0 and not np.signbit(val(0x00))
    assert val(0x80) == 0.0 and np.signbit(val(0x80))
    assert np.isnan(val(0x7F)) and np.isnan(val(0xFF))
    # exactly two NaN codes, no infinities
    all_vals = codecs.e4m3_to_f64(np.arange(256, dtype=np.uint8))
    assert np.isnan(all_vals).sum() == 2
    assert not np.isinf(all_vals).any()


def test_e4m3_encode_round_trips_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    back = codecs.f64_to_e4m3(codecs.e4m3_to_f64(codes))
    assert np.array_equal(back, codes)


def test_e4m3_encode_ties_go_to_even_code():
    pos = codecs.e4m3_to_f64(np.arange(0x7F, dtype=np.uint8))
    mids = (pos[:-1] + pos[1:]) / 2.0
    got = codecs.f64_to_e4m3(mids)
    lo = np.arange(0x7E, dtype=np.int64)
    expect = np.where(lo % 2 == 0, lo, lo + 1)
    assert np.array_equal(got.astype(np.int64), expect)
    # just off the midpoint rounds to the nearer neighbour
    up = codecs.f64_to_e4m3(np.nextafter(mids, np.inf))
    down = codecs.f64_to_e4m3(np.nextafter(mids, -np.inf))
    assert np.array_equal(up.astype(np.int64), lo + 1)
    assert np.array_equal(down.astype(np.int64), lo)


def test_e4m3_encode_matches_library_in_range():
    rng = np.random.default_rng(7)
    x = np.concatenate([
        rng.standard_normal(20000) * 50.0,
        rng.standard_normal(20000) * 1e-2,
        rng.uniform(-447.9, 447.9, 20000),
    ]).astype(np.float32)
    pos = codecs.e4m3_to_f64(np.arange(0x7F, dtype=np.uint8))
    mids = ((pos[:-1] + pos[1:]) / 2.0).astype(np.float32)
    x = np.concatenate([x, mids, -mids])
    ours = codecs.f64_to_e4m3(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_e4m3_saturation_and_nan():
    got = codecs.f64_to_e4m3(np.array([448.0, 460.0, 464.0, 1e30, np.inf, -500.0, -np.inf, np.nan, -0.0, -1e-30]))
    assert list(got) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE, 0x7F, 0x80, 0x80]


def test_quantize_uses_one_correctly_rounded_f32_division():
    rng = np.random.default_rng(11)
    x = rng.standard_normal(50000).astype(np.float32)
    scale = np.float32(np.max(np.abs(x)) / 448.0)
    # f64 quotient rounded once to f32 is the correctly rounded f32 quotient
    q = (x.astype(np.float64) / np.float64(scale)).astype(np.float32)
    expect = torch.from_numpy(q).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codecs.quantize_e4m3(x, scale), expect)


@pytest.mark.parametrize("dtype,tdtype", [("bf16", torch.bfloat16), ("f16", torch.float16)])
def test_16bit_decode_matches_library(dtype, tdtype):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = codecs.bits_to_f64(bits, dtype)
    ref = torch.from_numpy(bits.view(np.int16)).view(tdtype).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])


def test_bf16_closed_forms():
    val = lambda b: float(codecs.bits_to_f64(np.array([b], np.uint16), "bf16")[0])
    assert val(0x3F80) == 1.0
    assert val(0xC000) == -2.0
    assert val(0x7F7F) == (2 - 2 ** -7) * 2.0 ** 127
    assert val(0x0001) == 2.0 ** -133
    assert np.isinf(val(0x7F80))


def test_f32_decode_is_identity():
    x = np.random.default_rng(3).standard_normal(1000).astype(np.float32)
    assert np.array_equal(codecs.bits_to_f64(x.view(np.uint32), "f32"), x.astype(np.float64))
