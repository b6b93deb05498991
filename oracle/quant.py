"""Calibration and fake-quantization steps of the quantized attention path.

NVIDIA blog "Optimizing FLUX.1 Kontext for Image Editing with Low-Precision
Quantization", section "Workflow and Quantization":
  * Q, K and V are quantized per-tensor FP8 or per-block FP4, as the quantization
    config chooses (first bullet); the FP8 and FP4 variants differ only in the
    precision of Q, K and V (paragraph after the bullets);
  * BMM1's inputs get an extra quantization to FP8 (second bullet) and BMM2 runs
    in per-tensor FP8 (fourth bullet); in Fig. 4 the inputs are block-FP4
    quantized while both BMMs are per-tensor FP8, and the quant nodes are
    FakeQuantize operations;
  * scales are fixed by post-training calibration (step 4 of the workflow list).

Readings where the page is silent: the calibrator is max |x| over the quantizer's
own input; the per-tensor FP8 scale is s = amax/448 with encode x * (448/amax);
FP4 blocks are 32 consecutive elements along the head dimension with an E8M0
scale 2^e, e = floor(log2(block amax)) - 2 (the OCP MX scale rule), clamped to
[-127, 127].
"""
from __future__ import annotations

import math

import numpy as np

from . import formats as F

FP4_BLOCK = 32


def amax(x) -> float:
    """Calibration statistic: max |x| over the whole tensor (a max calibrator)."""
    x = np.asarray(x)
    return float(np.max(np.abs(x.astype(np.float64)))) if x.size else 0.0


def fp8_scales(amax_value: float):
    """Per-tensor FP8 scale s = fl32(amax / 448) and its encode factor inv = fl32(448 / amax).

    A zero amax (an all-zero tensor) gives s = inv = 1.
    """
    a = np.float32(amax_value)
    if a == 0:
        return np.float32(1.0), np.float32(1.0)
    return np.float32(a / np.float32(F.E4M3_MAX)), np.float32(np.float32(F.E4M3_MAX) / a)


def fp8_codes(x_f32, inv) -> np.ndarray:
    """Per-tensor FP8 quantization: code = E4M3_RNE_sat(fl32(x * inv)); x is float32."""
    x = np.asarray(x_f32, dtype=np.float32)
    return F.e4m3_encode(x * np.float32(inv))       # float32 product, one IEEE rounding


def fp8_dequant(codes, s) -> np.ndarray:
    return F.e4m3_decode(codes) * np.float64(np.float32(s))


def e8m0_exponent(block_amax: float) -> int:
    """Shared block exponent e = floor(log2(amax)) - 2, clamped to [-127, 127]; amax 0 -> -127.

    floor(log2 a) comes from frexp (a = m * 2^E, 0.5 <= m < 1, so floor(log2 a) = E - 1).
    """
    if block_amax == 0.0:
        return -127
    _, E = math.frexp(block_amax)
    return max(-127, min(127, (E - 1) - 2))


def fp4_block_quant(x_f32, block: int = FP4_BLOCK):
    """Per-block FP4 fake-quant along the last axis.

    Returns (codes, scales, dq):
      codes  uint8 [..., d/2]: two E2M1 codes per byte, even element in the low nibble
      scales uint8 [..., d/block]: E8M0 byte e + 127 of each block
      dq     float32 [..., d]: E2M1(code) * 2^e (always exact in bf16)
    """
    x = np.asarray(x_f32, dtype=np.float32)
    d = x.shape[-1]
    if d % block:
        raise ValueError("d must be a multiple of the block size")
    xb = x.astype(np.float64).reshape(-1, d // block, block)
    amaxes = np.max(np.abs(xb), axis=-1)
    e = np.vectorize(e8m0_exponent, otypes=[np.int64])(amaxes) if amaxes.size else \
        np.zeros(amaxes.shape, np.int64)
    q = xb / np.ldexp(1.0, e)[..., None]            # exact: division by a power of two
    c = F.e2m1_encode(q)
    dq = F.e2m1_decode(c) * np.ldexp(1.0, e)[..., None]
    c = c.reshape(x.shape)
    codes = (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)
    scales = (e + 127).astype(np.uint8).reshape(x.shape[:-1] + (d // block,))
    return codes, scales, dq.reshape(x.shape).astype(np.float32)


def fp4_unpack(codes, scales, block: int = FP4_BLOCK) -> np.ndarray:
    """Dequantize packed E2M1 codes with their E8M0 scales (float64)."""
    codes = np.asarray(codes, dtype=np.uint8)
    c = np.stack([codes & 0xF, codes >> 4], axis=-1).reshape(codes.shape[:-1] + (-1,))
    v = F.e2m1_decode(c)
    s = F.e8m0_decode(np.repeat(np.asarray(scales), block, axis=-1))
    return v * s
