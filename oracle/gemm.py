"""Quantized projection GEMMs — TEST INFRASTRUCTURE ONLY (see the package docstring).

NVIDIA blog "Optimizing FLUX.1 Kontext for Image Editing with Low-Precision
Quantization": the transformer's time splits between the attention operator and
the GEMMs of its linear layers (section on where the time goes), and the
quantization config applies per-tensor FP8 or per-block FP4 to the model's
linear layers as post-training quantization ("Workflow and Quantization", the
quantization config and the PTQ paragraph).  The pages give no layer sizes; the
projections modelled here take the attention's own width H * d = 24 * 128 = 3072:
the QKV projection 3072 -> 3 * 3072 and the output projection 3072 -> 3072, with
one GEMM row per token.

Readings where the pages are silent:
  * C = A B^T with A the activations [M, K] (one row per token) and B the weights
    [N, K] (one row per output feature), both K-contiguous;
  * FP8 (W8A8): per-tensor E4M3 codes with the static scales of the attention path
    (s = amax / 448), C = s_a s_b sum_k E4M3(a_mk) E4M3(b_nk);
  * FP4: OCP MX E2M1 codes in blocks of 32 consecutive k with an E8M0 scale per
    block, for both operands (the layout `quant.fp4_block_quant` produces),
    C = sum_k dq(a)_mk dq(b)_nk.

Exactness.  Every E4M3 value is an integer multiple of 2^-9 below 2^18 * 2^-9, so a
product is an integer multiple of 2^-18 below 2^36 * 2^-18 and every partial sum of
K <= 2^17 products is an integer multiple of 2^-18 below 2^53 * 2^-18: the float64
sum is exact in any order.  E2M1 values are multiples of 1/2 up to 6; within one
32-block the products share the scale 2^(e_a + e_b), so each block's float64 sum is
exact, and the sum over blocks is exact while the blocks' scales stay within
2^(53 - 11) of each other (far wider than any data-derived scales).
"""
from __future__ import annotations

import numpy as np

from . import formats as F
from . import quant as Q


def gemm_fp8(a8, b8, s_a, s_b) -> np.ndarray:
    """C = s_a s_b (E4M3(a8) @ E4M3(b8)^T) in float64; a8 [M, K], b8 [N, K] uint8 codes."""
    a = F.e4m3_decode(np.asarray(a8, dtype=np.uint8))
    b = F.e4m3_decode(np.asarray(b8, dtype=np.uint8))
    if a.shape[-1] != b.shape[-1]:
        raise ValueError("K mismatch")
    return (a @ b.T) * (float(s_a) * float(s_b))


def gemm_mxfp4(a_codes, a_scales, b_codes, b_scales) -> np.ndarray:
    """C = dq(a) @ dq(b)^T in float64 from packed E2M1 codes [rows, K/2] (low nibble = even
    element) and E8M0 block scales [rows, K/32]."""
    a = Q.fp4_unpack(a_codes, a_scales)
    b = Q.fp4_unpack(b_codes, b_scales)
    if a.shape[-1] != b.shape[-1]:
        raise ValueError("K mismatch")
    return a @ b.T
