"""Element codecs for the KV cache -- test infrastructure only (oracle).

The pages name 16-bit KV caches and an 8-bit float KV cache ("AI Inference
Serving at Scale", section 6: FP8 halves the KV footprint; "vLLM &
High-Throughput Serving", section 5 engine arguments).  They do not define
the bit formats, so these follow the public format definitions:

* bfloat16: the upper 16 bits of an IEEE-754 binary32 value.
* FP8 E4M3 in the OCP "FN" variant: 1 sign bit, 4 exponent bits with bias
  7, 3 mantissa bits; exponent field 0 holds subnormals m/8 * 2**-6; the
  single pattern S.1111.111 is NaN; there are no infinities; the largest
  finite magnitude is 1.75 * 2**8 = 448.

* FP8 E5M2 (OCP): 1 sign bit, 5 exponent bits with bias 15, 2 mantissa
  bits; exponent field 0 holds subnormals m/4 * 2**-14; exponent field 31
  is infinity (mantissa 0) or NaN; the largest finite magnitude is
  1.75 * 2**15 = 57344.  The third page names this format for its FP8 KV
  cache ("vLLM & High-Throughput Serving", section 5, kv_cache_dtype).

* INT4: a signed 4-bit integer code c in -8..7, stored as its two's
  complement nibble, standing for ``c * scale``.  The first page names a
  4-bit integer KV cache ("AI Inference Serving at Scale", section 6:
  4-bit keys and values quadruple the requests one GPU holds) without its
  scheme; the reading here is the plain symmetric one with one float32
  scale per group, a group being one token's head vector of K (or of V)
  in one KV head: ``scale = absmax / 7`` and ``c = round(x / scale)``,
  nearest-even, so the encoder emits -7..7 (the pattern of -8 decodes but
  is never written).

Everything returns numpy float64, in which all these formats are exact.
"""

from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
E5M2_MAX = 57344.0
INT4_LEVEL = 7  # largest code magnitude the INT4 encoder emits


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns (uint16) to float64, exactly.

    A bfloat16 is the high half of a binary32, so placing the 16 bits in
    the top of a 32-bit word gives the identical binary32 value.
    """
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def e4m3_to_f64(codes: np.ndarray) -> np.ndarray:
    """Decode OCP E4M3FN codes (uint8) to float64, from the field layout."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    exp = (c >> 3) & 0xF
    man = (c & 0x7).astype(np.float64)
    normal = (1.0 + man / 8.0) * np.exp2(exp.astype(np.float64) - 7.0)
    subnormal = (man / 8.0) * 2.0 ** -6
    mag = np.where(exp == 0, subnormal, normal)
    mag = np.where((exp == 0xF) & ((c & 0x7) == 0x7), np.nan, mag)
    return sign * mag


def _e4m3_positive_table() -> tuple[np.ndarray, np.ndarray]:
    """All non-negative finite E4M3FN values in increasing order, with codes."""
    codes = np.arange(0, 0x7F, dtype=np.uint8)  # 0x7F is NaN
    return e4m3_to_f64(codes), codes


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """Round float values to E4M3FN codes: nearest, ties to even, saturating.

    Rounding is to the nearest representable magnitude; on an exact tie the
    code with an even mantissa (even last bit) wins, which is IEEE
    round-to-nearest-even.  Magnitudes above 448 saturate to 448 instead of
    becoming NaN; NaN input gives the NaN code with the input's sign.  The
    input is taken at its float64 value (callers pass the float32 quotient
    of value by scale, so the quotient's own rounding is binary32's).
    """
    x = np.asarray(x, dtype=np.float64)
    vals, codes = _e4m3_positive_table()
    mag = np.abs(x)
    neg = np.signbit(x)
    clipped = np.minimum(mag, E4M3_MAX)
    hi = np.searchsorted(vals, clipped, side="left")  # first vals >= clipped
    hi = np.minimum(hi, len(vals) - 1)
    lo = np.maximum(hi - 1, 0)
    d_hi = vals[hi] - clipped
    d_lo = clipped - vals[lo]
    pick_hi = d_hi < d_lo
    tie = d_hi == d_lo
    hi_even = (codes[hi] & 1) == 0
    pick_hi = np.where(tie, hi_even, pick_hi)
    out = np.where(pick_hi, codes[hi], codes[lo]).astype(np.uint8)
    out = np.where(vals[hi] == clipped, codes[hi], out).astype(np.uint8)
    out = out | np.where(neg, np.uint8(0x80), np.uint8(0)).astype(np.uint8)
    nan_code = np.where(neg, np.uint8(0xFF), np.uint8(0x7F)).astype(np.uint8)
    return np.where(np.isnan(x), nan_code, out).astype(np.uint8)


def e5m2_to_f64(codes: np.ndarray) -> np.ndarray:
    """Decode OCP E5M2 codes (uint8) to float64, from the field layout."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    exp = (c >> 2) & 0x1F
    man = (c & 0x3).astype(np.float64)
    normal = (1.0 + man / 4.0) * np.exp2(exp.astype(np.float64) - 15.0)
    subnormal = (man / 4.0) * 2.0 ** -14
    mag = np.where(exp == 0, subnormal, normal)
    mag = np.where(exp == 0x1F, np.where((c & 0x3) == 0, np.inf, np.nan), mag)
    return sign * mag


def e5m2_encode(x: np.ndarray) -> np.ndarray:
    """Round float values to E5M2 codes: nearest, ties to even, saturating.

    As ``e4m3_encode``: the nearest finite magnitude, an exact tie going to
    the code with the even last bit; magnitudes above 57344 (infinity
    included) saturate to 57344 -- the cache never stores an infinity;
    NaN gives the NaN code 0x7F with the input's sign.
    """
    x = np.asarray(x, dtype=np.float64)
    codes = np.arange(0, 0x7C, dtype=np.uint8)  # 0x7C is +inf
    vals = e5m2_to_f64(codes)
    mag = np.abs(x)
    neg = np.signbit(x)
    clipped = np.minimum(mag, E5M2_MAX)
    hi = np.searchsorted(vals, clipped, side="left")
    hi = np.minimum(hi, len(vals) - 1)
    lo = np.maximum(hi - 1, 0)
    d_hi = vals[hi] - clipped
    d_lo = clipped - vals[lo]
    pick_hi = np.where(d_hi == d_lo, (codes[hi] & 1) == 0, d_hi < d_lo)
    out = np.where(pick_hi, codes[hi], codes[lo]).astype(np.uint8)
    out = np.where(vals[hi] == clipped, codes[hi], out).astype(np.uint8)
    out = out | np.where(neg, np.uint8(0x80), np.uint8(0)).astype(np.uint8)
    nan_code = np.where(neg, np.uint8(0xFF), np.uint8(0x7F)).astype(np.uint8)
    return np.where(np.isnan(x), nan_code, out).astype(np.uint8)


def int4_encode(x: np.ndarray) -> tuple[np.ndarray, np.float32]:
    """Quantize one group (a token's head vector) to INT4 codes and a scale.

    ``scale = float32(absmax) / 7`` (one binary32 division, nearest-even),
    then each code is ``x / scale`` rounded once in binary32 and then to the
    nearest integer, ties to even, kept within -7..7.  An all-zero group
    gets scale 0 and zero codes.  Inputs must be finite.
    """
    x = np.asarray(x, dtype=np.float32)
    absmax = np.float32(np.max(np.abs(x))) if x.size else np.float32(0.0)
    scale = np.float32(absmax / np.float32(INT4_LEVEL))
    if scale == 0:
        return np.zeros(x.shape, dtype=np.int8), np.float32(0.0)
    quotient = (x / scale).astype(np.float32)
    codes = np.clip(np.rint(quotient), -INT4_LEVEL, INT4_LEVEL)
    return codes.astype(np.int8), scale


def int4_to_f64(codes: np.ndarray, scale) -> np.ndarray:
    """Value of INT4 codes (integers -8..7) under their float32 scale."""
    c = np.asarray(codes, dtype=np.int64).astype(np.float64)
    return c * np.float64(np.float32(scale))


def nibble_to_int4(n: np.ndarray) -> np.ndarray:
    """Two's complement 4-bit patterns (0..15) -> integers -8..7."""
    n = np.asarray(n, dtype=np.int64) & 0xF
    return np.where(n >= 8, n - 16, n)


def int4_to_nibble(c: np.ndarray) -> np.ndarray:
    """Integers -8..7 -> their two's complement 4-bit patterns."""
    c = np.asarray(c, dtype=np.int64)
    if np.any((c < -8) | (c > 7)):
        raise ValueError("INT4 code out of range")
    return (c & 0xF).astype(np.uint8)
