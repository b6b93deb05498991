"""Quantized attention, full-row (non-online) form, plus the variants that are reported.

NVIDIA blog "Optimizing FLUX.1 Kontext for Image Editing with Low-Precision
Quantization", section "Workflow and Quantization", bullets 2-4 and Fig. 4:
BMM1 = Q K^T on FP8 inputs with its output accumulated in higher precision;
softmax in FP32 with no quantization; BMM2 = P V with per-tensor FP8.

R3 (the gated reading of where BMM2's FP8 P scale sits; the page fixes neither
the tensor nor the value).  For query row i of one (batch, head):

  raw_ij = sum_k E4M3(q_ik) E4M3(k_jk)              exact (float64, see below)
  t_ij   = fl32(raw_ij * c1),  c1 = fl32(s_Q s_K sm_scale log2(e))
  M_i    = ceil(max_j t_ij)                          integer row offset
  p_ij   = fl32(exp2(t_ij - M_i))                    in (0, 1]; softmax numerator, FP32
  l_i    = fl32(sum_j p_ij)                          unquantized FP32 row sum
  cp_ij  = E4M3_RNE_sat(fl32(p_ij * 448))            static per-tensor FP8, s_P = 1/448
  acc_i  = sum_j E4M3(cp_ij) E4M3(v_j)               exact (float64)
  O_i    = fl32(acc_i * c2 / l_i),  c2 = fl32(s_V / 448)

so O = softmax(Q K^T sm_scale) V up to the quantization of Q, K, V and P.
Exactness of the two matrix products: every E4M3 value is an integer multiple
of 2^-9 with magnitude at most 448 < 2^9, so each product is an integer multiple
of 2^-18 below 2^36 units and any partial sum of fewer than 2^17 products stays
below 2^53 units: a float64 matrix product returns the exact sum in any order.
raw * c1 is formed in float64 and rounded once to float32 (in the rare case that
the float64 product itself rounds, this is a double rounding of at most 1 ulp).

R3 with a native MXFP4 BMM1 (a hardware-native variant, not the pages' numerics: the pages
keep both products in FP8).  Q and K stay in their per-block FP4 form (E2M1 codes with an E8M0
scale per 32 elements of d, the output of the FP4 fake-quantizer) and BMM1 multiplies the
dequantized values directly, without the per-tensor FP8 step:

  raw_ij = sum_k dq4(q)_ik dq4(k)_jk,  dq4 = E2M1 value * 2^(scale byte - 127)
  t_ij   = fl32(raw_ij * c1),  c1 = fl32(sm_scale log2(e))

and the rest as R3 (V, P in FP8).  raw is exact in float64: within one 32-block the products
share the scale 2^(e_q + e_k) and are multiples of 1/4 of it below 36, so each block's sum
is exact, and the four block sums of d = 128 are exact while their scales stay within
2^(53 - 13) of each other (data-derived block exponents differ by far less).

R1 (reported, not gated): the literal FakeQuantize on the normalized P = p/l with
a per-tensor scale s_P = amax_P / 448 calibrated over the whole P tensor.
FP64 reference (reported, not gated): softmax(Q K^T sm_scale) V on the
unquantized inputs, all in float64.
"""
from __future__ import annotations

import math

import numpy as np

from . import formats as F

LOG2E = 1.0 / math.log(2.0)
P_SCALE = 448.0


def constants(s_q, s_k, s_v, sm_scale):
    """c1 = fl32(s_Q s_K sm_scale log2 e) and c2 = fl32(s_V / 448), products in float64."""
    c1 = np.float32(float(np.float32(s_q)) * float(np.float32(s_k))
                    * float(np.float32(sm_scale)) * LOG2E)
    c2 = np.float32(float(np.float32(s_v)) / P_SCALE)
    return c1, c2


def r3_rows(Qv, Kv, Vv, c1, c2, quantize_p: bool = True):
    """R3 for a block of query rows of one (batch, head).

    Qv [R, d], Kv [N, d], Vv [N, d]: float64 operand values (the decoded E4M3 codes,
    unscaled).  c1, c2 as in the module docstring.  With quantize_p False the P
    quantizer is the identity (used to check the path against textbook attention).
    Returns (O float32 [R, d], M float64 [R], l float32 [R]).
    """
    raw = Qv @ Kv.T
    t = F.fl32(raw * float(c1)).astype(np.float64)
    M = np.ceil(np.max(t, axis=1, keepdims=True))
    p = F.fl32(np.exp2(t - M))
    l = F.fl32(np.sum(p.astype(np.float64), axis=1))
    if quantize_p:
        pv = F.e4m3_decode(F.e4m3_encode(p * np.float32(P_SCALE)))
    else:
        pv = p.astype(np.float64) * P_SCALE
    acc = pv @ Vv
    O = F.fl32(acc * float(c2) / l.astype(np.float64)[:, None])
    return O, M[:, 0], l


def attention_r3(q8, k8, v8, s_q, s_k, s_v, sm_scale, rows=None, chunk: int = 256):
    """R3 quantized attention from E4M3 codes.

    q8, k8, v8: uint8 [B, H, N, d] (V in its natural token-major layout).
    rows: optional 1-D array of query indices to evaluate (each row is independent).
    Returns (O float32 [B, H, R, d], M float64 [B, H, R], l float32 [B, H, R]).
    """
    B, H, N, d = q8.shape
    rows = np.arange(N) if rows is None else np.asarray(rows)
    c1, c2 = constants(s_q, s_k, s_v, sm_scale)
    O = np.empty((B, H, len(rows), d), np.float32)
    M = np.empty((B, H, len(rows)), np.float64)
    L = np.empty((B, H, len(rows)), np.float32)
    for b in range(B):
        for h in range(H):
            Kv = F.e4m3_decode(k8[b, h])
            Vv = F.e4m3_decode(v8[b, h])
            for r0 in range(0, len(rows), chunk):
                rr = rows[r0:r0 + chunk]
                Qv = F.e4m3_decode(q8[b, h, rr])
                O[b, h, r0:r0 + len(rr)], M[b, h, r0:r0 + len(rr)], L[b, h, r0:r0 + len(rr)] = \
                    r3_rows(Qv, Kv, Vv, c1, c2)
    return O, M, L


def attention_r3_mxfp4(q_codes, q_scales, k_codes, k_scales, v8, s_v, sm_scale, rows=None,
                       chunk: int = 256):
    """R3 with BMM1 on the FP4 block-quantized Q and K (see the module docstring).

    q_codes, k_codes: uint8 [B, H, N, d/2] packed E2M1 (even element in the low nibble);
    q_scales, k_scales: uint8 [B, H, N, d/32] E8M0; v8: uint8 [B, H, N, d] E4M3 codes of V
    (token-major) with per-tensor scale s_v.  Returns (O, M, l) like attention_r3.
    """
    from . import quant as Qz
    B, H, N = q_codes.shape[:3]
    d = 2 * q_codes.shape[3]
    rows = np.arange(N) if rows is None else np.asarray(rows)
    c1, c2 = constants(1.0, 1.0, s_v, sm_scale)
    O = np.empty((B, H, len(rows), d), np.float32)
    M = np.empty((B, H, len(rows)), np.float64)
    L = np.empty((B, H, len(rows)), np.float32)
    for b in range(B):
        for h in range(H):
            Kv = Qz.fp4_unpack(k_codes[b, h], k_scales[b, h])
            Vv = F.e4m3_decode(v8[b, h])
            for r0 in range(0, len(rows), chunk):
                rr = rows[r0:r0 + chunk]
                Qv = Qz.fp4_unpack(q_codes[b, h, rr], q_scales[b, h, rr])
                O[b, h, r0:r0 + len(rr)], M[b, h, r0:r0 + len(rr)], L[b, h, r0:r0 + len(rr)] = \
                    r3_rows(Qv, Kv, Vv, c1, c2)
    return O, M, L


def attention_r1(q8, k8, v8, s_q, s_k, s_v, sm_scale, amax_p=None, rows=None):
    """R1: FakeQuantize on the normalized FP32 P with a calibrated per-tensor scale.

    P_ij = fl32(p_ij / l_i) with p, l as in R3 (the max shift cancels in P up to rounding);
    s_P = fl32(amax_P / 448) over the whole tensor; O = (E4M3(P / s_P) s_P) @ (E4M3(v) s_V).
    amax_P: the static calibrated maximum of P; None calibrates it on these inputs (max of P
    over every row of every head, which needs rows=None).  rows: optional query rows to
    evaluate (each row needs all keys, not the other rows).
    Returns (O float32 [B, H, R, d], amax_p).
    """
    B, H, N, d = q8.shape
    rows = np.arange(N) if rows is None else np.asarray(rows)
    if amax_p is None and len(rows) != N:
        raise ValueError("calibrating amax_P needs every row")
    c1, _ = constants(s_q, s_k, s_v, sm_scale)
    Ps = []
    for b in range(B):
        for h in range(H):
            raw = F.e4m3_decode(q8[b, h, rows]) @ F.e4m3_decode(k8[b, h]).T
            t = F.fl32(raw * float(c1)).astype(np.float64)
            p = F.fl32(np.exp2(t - np.ceil(np.max(t, axis=1, keepdims=True))))
            l = F.fl32(np.sum(p.astype(np.float64), axis=1))
            Ps.append(p / l[:, None])                      # float32 / float32 -> float32
    if amax_p is None:
        amax_p = max(float(np.max(P)) for P in Ps)
    s_p = np.float32(np.float32(amax_p) / np.float32(P_SCALE))
    inv_p = np.float32(np.float32(P_SCALE) / np.float32(amax_p))
    O = np.empty((B, H, len(rows), d), np.float32)
    for i, P in enumerate(Ps):
        b, h = divmod(i, H)
        pq = F.e4m3_decode(F.e4m3_encode(P * inv_p)) * float(s_p)
        vv = F.e4m3_decode(v8[b, h]) * float(np.float32(s_v))
        O[b, h] = F.fl32(pq @ vv)
    return O, amax_p


def attention_fp64(q, k, v, sm_scale, rows=None):
    """Unquantized softmax(q k^T sm_scale) v in float64; q, k, v float arrays [B, H, N, d]."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    rows = np.arange(q.shape[2]) if rows is None else np.asarray(rows)
    B, H = q.shape[:2]
    O = np.empty((B, H, len(rows), q.shape[3]), np.float64)
    for b in range(B):
        for h in range(H):
            s = (q[b, h, rows] @ k[b, h].T) * float(sm_scale)
            s = s - np.max(s, axis=1, keepdims=True)
            e = np.exp(s)
            O[b, h] = (e / np.sum(e, axis=1, keepdims=True)) @ v[b, h]
    return O
