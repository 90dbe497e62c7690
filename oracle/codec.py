"""1-byte KV element codes for the oracle (test infrastructure only).

The pages say only that the KV cache may be stored as INT8 or FP8, one byte per
element, halving FP16's footprint ("从KV Cache到vLLM" (xxqk.cn) §2.2 and §2.3).
They fix neither the FP8 variant nor the integer code, so the readings are:

* FP8 is OCP E4M3FN: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits,
  no infinities, a single NaN pattern per sign (S.1111.111), largest finite
  value 448, subnormals k * 2**-9 for k = 1..7.
* INT8 is symmetric: codes -127..127 (-128 unused), value = code.

Both decoders are exact in float64.  The encoders round to nearest with ties to
even and saturate (FP8 to +-448, INT8 to +-127).
"""
import numpy as np

_E4M3_BIAS = 7
_E4M3_MAX = 448.0


def _e4m3fn_value(code):
    """Value of one E4M3FN code, straight from the field definition."""
    sign = -1.0 if code & 0x80 else 1.0
    exp_field = (code >> 3) & 0xF
    mant_field = code & 0x7
    if exp_field == 0xF and mant_field == 0x7:
        return np.nan
    if exp_field == 0:  # subnormal: 0.mmm * 2**(1 - bias)
        return sign * (mant_field / 8.0) * 2.0 ** (1 - _E4M3_BIAS)
    return sign * (1.0 + mant_field / 8.0) * 2.0 ** (exp_field - _E4M3_BIAS)


_E4M3_TABLE = np.array([_e4m3fn_value(c) for c in range(256)], dtype=np.float64)
# Non-negative finite codes 0x00..0x7E are increasing in value.
_E4M3_POS_VALUES = _E4M3_TABLE[:0x7F]


def e4m3fn_decode(codes):
    """uint8 codes (any shape) -> float64 values."""
    codes = np.asarray(codes)
    if codes.dtype != np.uint8:
        raise TypeError("e4m3fn codes must be uint8")
    return _E4M3_TABLE[codes]


def e4m3fn_encode(x):
    """float values -> uint8 E4M3FN codes, round-to-nearest-even, saturating.

    Each magnitude is placed between its two neighbouring representable values;
    the nearer wins, and on an exact tie the code with an even mantissa (an even
    code, since the mantissa is the low bits) wins.  Magnitudes above 448
    saturate to 448; NaN maps to 0x7F.
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    a_clamped = np.minimum(a, _E4M3_MAX)
    hi = np.searchsorted(_E4M3_POS_VALUES, a_clamped, side="left")  # first value >= a
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    exact = _E4M3_POS_VALUES[hi] == a_clamped
    d_lo = a_clamped - _E4M3_POS_VALUES[lo]
    d_hi = _E4M3_POS_VALUES[hi] - a_clamped
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    mag = np.where(exact, hi, np.where(pick_hi, hi, lo)).astype(np.uint8)
    code = mag | np.where(np.signbit(x), 0x80, 0).astype(np.uint8)
    code = np.where(np.isnan(x), np.uint8(0x7F), code)
    return code.astype(np.uint8)


def int8_decode(codes):
    codes = np.asarray(codes)
    if codes.dtype != np.int8:
        raise TypeError("int8 codes must be int8")
    return codes.astype(np.float64)


def int8_encode(x):
    """float values -> int8 codes: round half to even, clip to [-127, 127]."""
    return np.clip(np.rint(np.asarray(x, dtype=np.float64)), -127, 127).astype(np.int8)
