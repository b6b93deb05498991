"""SVD-Quant in FP4 for a projection GEMM — TEST INFRASTRUCTURE ONLY (see the package docstring).

NVIDIA blog "Optimizing FLUX.1 Kontext for Image Editing with Low-Precision Quantization",
section "Workflow and Quantization": besides post-training quantization in FP8 and in FP4, the
work covers SVD-Quant in FP4.  The page names the method and gives no step of it; the reading
here is the method's plainest form for one linear layer C = A W^T (A [M, K] activations, one
row per token; W [N, K] weights, both K-contiguous, as in `gemm`): a low-rank part of W stays
in 16-bit, and only the remainder goes to FP4.

Weights (offline, once):
  W = U S V^T                                   float64 SVD of the bf16 weights
  L_up   = bf16(U[:, :r] S[:r])                 [N, r]   16-bit factors, each value rounded
  L_down = bf16(V[:, :r]^T)                     [r, K]   once from float64 (nearest even)
  R      = bf16(W - L_up L_down)                [N, K]   the residual, float64 then one rounding
  R4     = FP4 block quantization of R          E2M1 + E8M0 per 32 along K (quant.fp4_block_quant)
Forward (every call):
  A4     = FP4 block quantization of A
  T      = bf16(A L_down^T)                     [M, r]   the 16-bit branch's down-projection
  C      = fl32(dq(A4) dq(R4)^T + T L_up^T)     float32 output

Readings where the page is silent: the FP4 format is the one of the FP4 variant (MXFP4, as in
`gemm.gemm_mxfp4`); the 16-bit type is bf16; no activation smoothing (the synthetic weights
carry their outliers as a planted low-rank component, see `workloads.lowrank_weight_bits`);
T is rounded to bf16 because the branch's up-projection multiplies 16-bit operands.

Exactness.  dq(A4) dq(R4)^T is exact in float64 (the argument of `gemm`).  A L_down^T: bf16
products carry 16 significant bits and the float64 sum keeps every bit while the products of a
row stay within 2^37 of each other, far wider than the data's range.  T L_up^T is r bf16
products per element, exact in float64.  So C is one rounding of the exact sum.
"""
from __future__ import annotations

import numpy as np

from . import formats as F
from . import gemm as G
from . import quant as Q


def bf16_round(x) -> np.ndarray:
    """Round float64 values to the nearest bf16 value (ties to even), returned as float64.

    x = m 2^e with m in [0.5, 1) (frexp); bf16 keeps 8 significant bits, so m becomes the
    nearest multiple of 2^-8 (numpy's round: halves to even).  The data here stay in bf16's
    normal range; values at or beyond its overflow are not expected and are rejected."""
    x = np.asarray(x, np.float64)
    m, e = np.frexp(x)
    y = np.ldexp(np.round(m * 256.0) / 256.0, e)
    if not np.all(np.isfinite(y)) or np.any(np.abs(y) > 3.3895313892515355e38):
        raise ValueError("value outside bf16's finite range")
    return y


def bf16_bits(x) -> np.ndarray:
    """bf16 bit patterns (uint16) of values already on the bf16 grid."""
    return F.f32_to_bf16_bits_exact(np.asarray(x, np.float32))


def factorize(w, rank: int):
    """Rank-r 16-bit factors of W [N, K] from its float64 SVD: (L_up [N, r], L_down [r, K]) as
    float64 arrays of bf16 values.  rank = 0 gives empty factors."""
    w = np.asarray(w, np.float64)
    N, K = w.shape
    if not 0 <= rank <= min(N, K):
        raise ValueError("rank out of range")
    if rank == 0:
        return np.zeros((N, 0)), np.zeros((0, K))
    U, S, Vt = np.linalg.svd(w, full_matrices=False)
    return bf16_round(U[:, :rank] * S[:rank]), bf16_round(Vt[:rank])


def residual(w, l_up, l_down) -> np.ndarray:
    """R = bf16(W - L_up L_down), float64 values on the bf16 grid."""
    return bf16_round(np.asarray(w, np.float64) - np.asarray(l_up) @ np.asarray(l_down))


def quantize_weights(w, rank: int):
    """The offline weight steps: (L_up, L_down, R, R codes, R scales)."""
    l_up, l_down = factorize(w, rank)
    r = residual(w, l_up, l_down)
    r_codes, r_scales, _ = Q.fp4_block_quant(r.astype(np.float32))
    return l_up, l_down, r, r_codes, r_scales


def down_projection(a, l_down) -> np.ndarray:
    """T = bf16(A L_down^T) [M, r] (float64 values on the bf16 grid)."""
    a = np.asarray(a, np.float64)
    if l_down.shape[0] == 0:
        return np.zeros((a.shape[0], 0))
    return bf16_round(a @ np.asarray(l_down, np.float64).T)


def forward(a, l_up, l_down, r_codes, r_scales, branch: bool = True):
    """C = fl32(dq(A4) dq(R4)^T + T L_up^T) for bf16 activations A [M, K] (float values).

    Returns (C float32 [M, N], T [M, r]).  branch=False drops the 16-bit branch (C is then
    the MXFP4 GEMM of A and the residual alone)."""
    a = np.asarray(a, np.float32)
    a_codes, a_scales, _ = Q.fp4_block_quant(a)
    c = G.gemm_mxfp4(a_codes, a_scales, r_codes, r_scales)
    t = down_projection(a, l_down)
    if branch and t.shape[1]:
        c = c + t @ np.asarray(l_up, np.float64).T
    return F.fl32(c), t
