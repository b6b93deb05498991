"""Number formats by their definitions: every code is decoded from its bit fields,
and encoding is a nearest-value search over the decoded set.

E4M3 follows the OCP 8-bit floating point specification ("E4M3FN"): 1 sign bit,
4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 is subnormal
(m/8 * 2^-6); S.1111.111 is NaN; there are no infinities; the largest finite
magnitude is 448.

E2M1 and E8M0 follow the OCP Microscaling (MX) specification v1.0: E2M1 has
1 sign bit, 2 exponent bits with bias 1 and 1 mantissa bit (magnitudes
0, 0.5, 1, 1.5, 2, 3, 4, 6); E8M0 is an unsigned biased exponent, 2^(byte-127),
with 0xFF as NaN.

Encoders round to nearest, with ties going to the code whose least significant
bit is 0 (round-half-to-even on the code), saturate to the largest finite
magnitude, and keep the sign bit of the input (so -0 and small negative values
encode to the negative-zero code).

The NVIDIA blog "Optimizing FLUX.1 Kontext for Image Editing with Low-Precision
Quantization" (section "Workflow and Quantization") names FP8 and FP4 without a
bit layout; E4M3 for FP8 and E2M1 with E8M0 block scales for FP4 are the
readings used here.
"""
from __future__ import annotations

import math

import numpy as np

E4M3_MAX = 448.0
E2M1_MAX = 6.0


def _e4m3_decode_one(code: int) -> float:
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return sign * math.ldexp(m / 8.0, 1 - 7)
    return sign * math.ldexp(1.0 + m / 8.0, e - 7)


def _e2m1_decode_one(code: int) -> float:
    sign = -1.0 if code & 0x8 else 1.0
    e = (code >> 1) & 0x3
    m = code & 0x1
    if e == 0:
        return sign * (m * 0.5)
    return sign * math.ldexp(1.0 + m / 2.0, e - 1)


E4M3_TABLE = np.array([_e4m3_decode_one(c) for c in range(256)], dtype=np.float64)
E2M1_TABLE = np.array([_e2m1_decode_one(c) for c in range(16)], dtype=np.float64)

# Non-negative finite magnitudes in code order; both sets are increasing in the code.
_E4M3_MAGS = E4M3_TABLE[:0x7F]          # codes 0x00 .. 0x7E
_E2M1_MAGS = E2M1_TABLE[:0x8]           # codes 0x0 .. 0x7


def _nearest_code(a: np.ndarray, mags: np.ndarray) -> np.ndarray:
    """Index of the value in increasing `mags` nearest to each a >= 0; ties to the even index;
    values beyond the last magnitude saturate to it."""
    hi = np.searchsorted(mags, a, side="left")           # mags[hi-1] < a <= mags[hi]
    hi = np.clip(hi, 1, len(mags) - 1)
    lo = hi - 1
    d_lo = a - mags[lo]
    d_hi = mags[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    idx = np.where(pick_hi, hi, lo)
    idx = np.where(a <= mags[0], 0, idx)
    idx = np.where(a >= mags[-1], len(mags) - 1, idx)
    return idx


def e4m3_encode(x) -> np.ndarray:
    """E4M3 codes of real values x (any float dtype), RNE, saturating at +-448, sign kept."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    code = _nearest_code(np.where(np.isnan(a), 0.0, a), _E4M3_MAGS).astype(np.uint8)
    code = np.where(np.isnan(a), np.uint8(0x7F), code).astype(np.uint8)
    return code | (np.signbit(x).astype(np.uint8) << 7)


def e4m3_decode(codes) -> np.ndarray:
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def e2m1_encode(x) -> np.ndarray:
    """E2M1 codes (0..15) of real values x, RNE on the code, saturating at +-6, sign kept."""
    x = np.asarray(x, dtype=np.float64)
    code = _nearest_code(np.abs(x), _E2M1_MAGS).astype(np.uint8)
    return code | (np.signbit(x).astype(np.uint8) << 3)


def e2m1_decode(codes) -> np.ndarray:
    return E2M1_TABLE[np.asarray(codes, dtype=np.uint8)]


def e8m0_decode(byte) -> np.ndarray:
    b = np.asarray(byte, dtype=np.int64)
    return np.where(b == 0xFF, np.nan, np.ldexp(1.0, b - 127))


def fl32(x) -> np.ndarray:
    """Round to IEEE binary32, nearest even."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def bf16_bits_to_f32(bits) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16_bits_exact(x) -> np.ndarray:
    """bf16 bits of float32 values that are exactly representable in bf16 (raises otherwise)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    if np.any(u & 0xFFFF):
        raise ValueError("value not representable in bf16")
    return (u >> 16).astype(np.uint16)
