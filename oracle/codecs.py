"""Element codecs for KV-pool storage types, written from the format definitions.

TEST INFRASTRUCTURE ONLY (see the package docstring).

A KV pool stores raw element bits.  The oracle never trusts a vendor conversion
for the values it checks against: every stored element is decoded from its
bits into float64 here, from the definition of its format.

Formats
  f32   IEEE-754 binary32.
  f16   IEEE-754 binary16 (NumPy's float16 is an exact implementation).
  bf16  the upper 16 bits of a binary32 (sign, 8 exponent bits, 7 mantissa
        bits), so decoding is "shift left by 16 and read as binary32".
  fp8   OCP 8-bit "E4M3" (the variant without infinities): 1 sign bit,
        4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 encodes
        subnormals M/8 * 2^-6; the all-ones pattern S.1111.111 is NaN; there
        is no infinity, so the largest finite magnitude is 1.75 * 2^8 = 448.

The pages use FP8 only as "1 byte per element plus scales" ([OT] "Quantized
KV": real FP8 caches also store quantization scales).  The reading taken here:
one fp32 scale per tensor (one for K, one for V); the stored code c represents
decode(c) * scale; a value x is stored as encode(x / scale), where the division
is one correctly-rounded binary32 division and encode rounds to the nearest
E4M3 value (ties to an even mantissa), saturating finite overflow to +-448 and
mapping NaN to 0x7F.
"""

import numpy as np

E4M3_MAX = 448.0


def bits_to_f64(raw: np.ndarray, dtype: str) -> np.ndarray:
    """Decode stored element bits to float64.

    raw: uint32 (f32), uint16 (f16 / bf16) or uint8 (fp8) array of bits.
    """
    if dtype == "f32":
        with np.errstate(invalid="ignore"):
            return np.ascontiguousarray(raw, dtype=np.uint32).view(np.float32).astype(np.float64)
    if dtype == "f16":
        return np.ascontiguousarray(raw, dtype=np.uint16).view(np.float16).astype(np.float64)
    if dtype == "bf16":
        widened = np.ascontiguousarray(raw, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        with np.errstate(invalid="ignore"):
            return widened.view(np.float32).astype(np.float64)
    if dtype == "fp8":
        return e4m3_to_f64(np.ascontiguousarray(raw, dtype=np.uint8))
    raise ValueError(f"unknown storage dtype {dtype!r}")


def e4m3_to_f64(codes: np.ndarray) -> np.ndarray:
    """Value of each OCP E4M3 code, straight from sign / exponent / mantissa."""
    codes = np.asarray(codes, dtype=np.uint8)
    sign = (codes >> 7).astype(np.int64)
    exp_field = ((codes >> 3) & 0xF).astype(np.int64)
    mant = (codes & 0x7).astype(np.int64)
    subnormal = mant / 8.0 * 2.0 ** -6
    normal = (1.0 + mant / 8.0) * np.power(2.0, (exp_field - 7).astype(np.float64))
    mag = np.where(exp_field == 0, subnormal, normal)
    val = np.where(sign == 1, -mag, mag)
    val = np.where((exp_field == 15) & (mant == 7), np.nan, val)
    return val.astype(np.float64)


# All finite non-negative E4M3 values, indexed by their code 0x00..0x7E.  The
# codes are ordered exactly like the values, so "nearest code" is a search.
_E4M3_NONNEG = e4m3_to_f64(np.arange(0x7F, dtype=np.uint8))


def f64_to_e4m3(y: np.ndarray) -> np.ndarray:
    """Round each value to the nearest E4M3 code: ties to even, saturating.

    y: float values that are exactly representable in float64 (the callers pass
    binary32 results).  NaN -> 0x7F; |y| >= 448 (including inf) -> +-448; the
    sign of zero and of values that round to zero is kept.
    """
    y = np.asarray(y, dtype=np.float64)
    flat = y.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint8)
    mag = np.abs(flat)
    neg = np.signbit(flat)
    nan = np.isnan(flat)
    sat = (~nan) & (mag >= E4M3_MAX)
    # Nearest of the two neighbouring representable magnitudes.
    hi = np.searchsorted(_E4M3_NONNEG, np.where(nan | sat, 0.0, mag), side="left")
    hi = np.clip(hi, 0, 0x7E)
    lo = np.clip(hi - 1, 0, 0x7E)
    d_hi = np.abs(_E4M3_NONNEG[hi] - mag)
    d_lo = np.abs(mag - _E4M3_NONNEG[lo])
    pick_lo = (d_lo < d_hi) | ((d_lo == d_hi) & (lo % 2 == 0))
    code = np.where(pick_lo, lo, hi).astype(np.uint8)
    code = np.where(sat, np.uint8(0x7E), code)
    code = np.where(neg, code | np.uint8(0x80), code)
    code = np.where(nan, np.uint8(0x7F), code)
    out[:] = code
    return out.reshape(y.shape)


def quantize_e4m3(x_f32: np.ndarray, scale: float) -> np.ndarray:
    """Store binary32 values into E4M3 codes with one per-tensor fp32 scale.

    The division x / scale is a single IEEE binary32 division (NumPy float32
    division is correctly rounded), then round-to-nearest-even into E4M3.
    """
    x32 = np.asarray(x_f32, dtype=np.float32)
    s32 = np.float32(scale)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        y = (x32 / s32).astype(np.float32)
    return f64_to_e4m3(y.astype(np.float64))
