"""Python binding of libkq, the quantized-SDPA library for MI355X (gfx950).

Thin ctypes marshalling over the C ABI declared in include/kq.h: every function below has
the name of the C entry point it calls, checks that tensors are contiguous device tensors
of the expected dtype and size, and passes raw pointers plus the current HIP stream.  All
arithmetic runs in the library's HIP kernels (or, for the two host-only helpers, in its
C code).  PyTorch supplies device memory and streams only.

The library must be built (``python -m precision_quantized_attention_amd.build`` or
``__graft_entry__.build()``); importing works without it, but every call raises
``KQError`` if ``libkq.so`` is missing.  There is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

__all__ = ["KQError", "LIB_PATH", "load", "KQ_LAYOUT_ROWS", "KQ_LAYOUT_TRANSPOSED",
           "kq_status_string", "kq_vt_ld", "kq_fp8_scales_from_amax", "kq_rope3_table",
           "kq_amax_calibrate", "kq_quantize_fp8_tensor", "kq_quantize_fp4_block",
           "kq_attn_quant_fwd", "kq_attn_workspace_size", "kq_attn_quant_fwd_ws",
           "kq_attn_quant_fwd_noalloc", "kq_attn_quant_fwd_qbf16",
           "kq_attn_mxfp4_fwd", "kq_attn_r1_stats", "kq_attn_r1_amax", "kq_attn_r1_fwd",
           "kq_gemm_fp8", "kq_gemm_mxfp4", "kq_gemm_fp8_bf16", "kq_gemm_mxfp4_bf16",
           "kq_svdquant_down", "kq_gemm_mxfp4_svdquant", "kq_gemm_mxfp4_svdquant_bf16",
           "kq_svdquant_factorize", "kq_svdquant_activations"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkq.so")
KQ_LAYOUT_ROWS = 0
KQ_LAYOUT_TRANSPOSED = 1


class KQError(RuntimeError):
    pass


class _Rope3(ctypes.Structure):
    _fields_ = [("cos_sin", ctypes.c_void_p), ("n_tokens", ctypes.c_int64)]


_lib = None

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I = ctypes.c_int
_F = ctypes.c_float

_SIGNATURES = {
    "kq_status_string": ([_I], ctypes.c_char_p),
    "kq_vt_ld": ([_I64], _I64),
    "kq_fp8_scales_from_amax": ([_F, ctypes.POINTER(_F), ctypes.POINTER(_F)], _I),
    "kq_rope3_table": ([_P, _I64, ctypes.c_double, _P], _I),
    "kq_amax_calibrate": ([_P, _I64, _P, _P], _I),
    "kq_quantize_fp8_tensor": ([_P, _I64, _I, _I64, _F, _P, _I, _P], _I),
    "kq_quantize_fp4_block": ([_P, _I64, _I, _P, _P, _P, _P, _F, ctypes.POINTER(_Rope3), _P],
                              _I),
    "kq_attn_quant_fwd": ([_P, _P, _P, _I, _I, _I, _I, _I, _F, _F, _F, _F, _P, _P, _P], _I),
    "kq_attn_workspace_size": ([_I, _I, _I, _I, ctypes.POINTER(ctypes.c_size_t)], _I),
    "kq_attn_quant_fwd_ws": ([_P, _P, _P, _I, _I, _I, _I, _I, _F, _F, _F, _F, _P, _P, _P,
                              ctypes.c_size_t, _P], _I),
    "kq_attn_quant_fwd_noalloc": ([_P, _P, _P, _I, _I, _I, _I, _I, _F, _F, _F, _F, _P, _P, _P],
                                  _I),
    "kq_attn_quant_fwd_qbf16": ([_P, _F, _P, _P, _I, _I, _I, _I, _I, _F, _F, _F, _F, _P, _P, _P,
                                 ctypes.c_size_t, _P], _I),
    "kq_attn_mxfp4_fwd": ([_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _F, _P, _P, _P,
                           ctypes.c_size_t, _P], _I),
    "kq_attn_r1_stats": ([_P, _P, _P, _I, _I, _I, _I, _I, _F, _F, _F, _F, _P, _P,
                          ctypes.c_size_t, _P], _I),
    "kq_attn_r1_amax": ([_P, _I64, _P, _P], _I),
    "kq_attn_r1_fwd": ([_P, _P, _P, _I, _I, _I, _I, _I, _F, _F, _F, _F, _F, _P, _P, _P,
                        ctypes.c_size_t, _P], _I),
    "kq_gemm_fp8": ([_P, _P, _I64, _I64, _I64, _F, _F, _P, _P], _I),
    "kq_gemm_mxfp4": ([_P, _P, _P, _P, _I64, _I64, _I64, _P, _P], _I),
    "kq_gemm_fp8_bf16": ([_P, _P, _I64, _I64, _I64, _F, _F, _P, _P], _I),
    "kq_gemm_mxfp4_bf16": ([_P, _P, _P, _P, _I64, _I64, _I64, _P, _P], _I),
    "kq_svdquant_down": ([_P, _P, _I64, _I64, _I, _P, _P], _I),
    "kq_svdquant_factorize": ([_P, _I64, _I64, _I, _P, _P, _P], _I),
    "kq_svdquant_activations": ([_P, _P, _I64, _I64, _I, _P, _P, _P, _P], _I),
    "kq_gemm_mxfp4_svdquant": ([_P, _P, _P, _P, _I64, _I64, _I64, _P, _P, _I, _P, _P], _I),
    "kq_gemm_mxfp4_svdquant_bf16": ([_P, _P, _P, _P, _I64, _I64, _I64, _P, _P, _I, _P, _P], _I),
}


def load():
    """Load libkq.so (once) and declare its signatures; raises KQError if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise KQError(f"{LIB_PATH} is not built; run precision_quantized_attention_amd.build")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGNATURES.items():
            f = getattr(lib, name)
            f.argtypes = args
            f.restype = res
        _lib = lib
    return _lib


def _check(status: int, what: str):
    if status != 0:
        msg = load().kq_status_string(status).decode()
        raise KQError(f"{what}: {msg} ({status})")


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _dev(t, dtype, name):
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise KQError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise KQError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise KQError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _opt(t, dtype, name):
    return None if t is None else _dev(t, dtype, name)


# ------------------------------------------------------------------ host helpers

def kq_status_string(status: int) -> str:
    return load().kq_status_string(status).decode()


def kq_vt_ld(n_tokens: int) -> int:
    return int(load().kq_vt_ld(n_tokens))


def kq_fp8_scales_from_amax(amax: float):
    """(scale, inv_scale) as numpy float32 from a calibrated amax (host-only C helper)."""
    s = _F()
    inv = _F()
    _check(load().kq_fp8_scales_from_amax(float(amax), ctypes.byref(s), ctypes.byref(inv)),
           "kq_fp8_scales_from_amax")
    return np.float32(s.value), np.float32(inv.value)


def kq_rope3_table(positions, theta: float = 10000.0) -> np.ndarray:
    """float32 [N, 64, 2] (cos, sin) table for int32 positions [N, 3] (host-only C helper)."""
    pos = np.ascontiguousarray(positions, dtype=np.int32)
    if pos.ndim != 2 or pos.shape[1] != 3:
        raise KQError("positions must be [N, 3]")
    out = np.empty((pos.shape[0], 64, 2), np.float32)
    _check(load().kq_rope3_table(pos.ctypes.data_as(_P), pos.shape[0], float(theta),
                                 out.ctypes.data_as(_P)), "kq_rope3_table")
    return out


# ------------------------------------------------------------------ device entry points

def kq_amax_calibrate(x, amax, stream=None):
    """amax[0] = max(amax[0], max|x|); x bf16 device tensor, amax float32 device tensor [1]."""
    import torch
    if amax.numel() != 1:
        raise KQError("amax must hold one float32")
    _check(load().kq_amax_calibrate(_dev(x, torch.bfloat16, "x"), x.numel(),
                                    _dev(amax, torch.float32, "amax"), _stream(stream)),
           "kq_amax_calibrate")


def kq_quantize_fp8_tensor(x, inv_scale: float, y, layout: int = KQ_LAYOUT_ROWS,
                           n_tokens: int = 0, stream=None):
    """E4M3 codes of x * inv_scale into y (uint8).  x: bf16 [..., d].
    layout KQ_LAYOUT_ROWS: y has x's shape.  KQ_LAYOUT_TRANSPOSED: x is [B, H, N, d] (or any
    [rows, d] with rows = BH * n_tokens) and y is [BH, d, kq_vt_ld(N)]."""
    import torch
    d = x.shape[-1]
    rows = x.numel() // d
    if layout == KQ_LAYOUT_ROWS:
        if y.numel() != x.numel():
            raise KQError("y must have as many elements as x")
    else:
        if n_tokens <= 0:
            n_tokens = x.shape[-2]
        if rows % n_tokens:
            raise KQError("rows must be a multiple of n_tokens")
        if y.numel() != (rows // n_tokens) * d * kq_vt_ld(n_tokens):
            raise KQError("y must be [B*H, d, kq_vt_ld(N)]")
    _check(load().kq_quantize_fp8_tensor(_dev(x, torch.bfloat16, "x"), rows, d, n_tokens,
                                         float(inv_scale), _dev(y, torch.uint8, "y"), layout,
                                         _stream(stream)), "kq_quantize_fp8_tensor")


def kq_quantize_fp4_block(x, codes, scales, dq=None, fp8=None, inv_scale8: float = 1.0,
                          rope=None, stream=None):
    """FP4 E2M1 block quantization of x (bf16 [..., d]).
    codes uint8 [..., d/2]; scales uint8 [..., d/32]; dq bf16 like x or None; fp8 uint8 like x
    or None; rope = (table float32 device tensor [N, 64, 2], N) or None."""
    import torch
    d = x.shape[-1]
    rows = x.numel() // d
    if codes.numel() != rows * d // 2 or scales.numel() != rows * d // 32:
        raise KQError("codes must be [rows, d/2] and scales [rows, d/32]")
    for t, nm in ((dq, "dq"), (fp8, "fp8")):
        if t is not None and t.numel() != x.numel():
            raise KQError(f"{nm} must have as many elements as x")
    rp = None
    if rope is not None:
        table, n_tok = rope
        if table.numel() != n_tok * d:
            raise KQError("rope table must be [N, d/2, 2]")
        rp = ctypes.byref(_Rope3(_dev(table, torch.float32, "rope table"), int(n_tok)))
    _check(load().kq_quantize_fp4_block(
        _dev(x, torch.bfloat16, "x"), rows, d, _dev(codes, torch.uint8, "codes"),
        _dev(scales, torch.uint8, "scales"), _opt(dq, torch.bfloat16, "dq"),
        _opt(fp8, torch.uint8, "fp8"), float(inv_scale8), rp, _stream(stream)),
        "kq_quantize_fp4_block")


def kq_attn_quant_fwd(q8, k8, v8t, s_q: float, s_k: float, s_v: float, sm_scale: float, o,
                      row_stats=None, v_layout: int = KQ_LAYOUT_TRANSPOSED, stream=None):
    """Fused quantized attention.  q8, k8: uint8 [B, H, N, d]; v8t: uint8 [B*H, d, kq_vt_ld(N)];
    o: float32 [B, H, N, d]; row_stats: float32 [B, H, N, 2] or None."""
    import torch
    B, H, N, d = q8.shape
    if tuple(k8.shape) != (B, H, N, d) or tuple(o.shape) != (B, H, N, d):
        raise KQError("k8 and o must match q8's shape")
    if v_layout == KQ_LAYOUT_TRANSPOSED and v8t.numel() != B * H * d * kq_vt_ld(N):
        raise KQError("v8t must be [B*H, d, kq_vt_ld(N)]")
    if row_stats is not None and row_stats.numel() != B * H * N * 2:
        raise KQError("row_stats must be [B, H, N, 2]")
    _check(load().kq_attn_quant_fwd(
        _dev(q8, torch.uint8, "q8"), _dev(k8, torch.uint8, "k8"), _dev(v8t, torch.uint8, "v8"),
        v_layout, B, H, N, d, float(s_q), float(s_k), float(s_v), float(sm_scale),
        _dev(o, torch.float32, "o"), _opt(row_stats, torch.float32, "row_stats"),
        _stream(stream)), "kq_attn_quant_fwd")


def kq_attn_workspace_size(B: int, H: int, N: int, d: int = 128) -> int:
    """Bytes of device workspace kq_attn_quant_fwd_ws uses for this shape on the current
    device (0: none needed)."""
    n = ctypes.c_size_t(0)
    _check(load().kq_attn_workspace_size(B, H, N, d, ctypes.byref(n)), "kq_attn_workspace_size")
    return int(n.value)


def kq_attn_quant_fwd_ws(q8, k8, v8t, s_q: float, s_k: float, s_v: float, sm_scale: float, o,
                         workspace, row_stats=None, v_layout: int = KQ_LAYOUT_TRANSPOSED,
                         stream=None):
    """kq_attn_quant_fwd with a device workspace (uint8 tensor of at least
    kq_attn_workspace_size bytes, or None) for the key split of the last round."""
    import torch
    B, H, N, d = q8.shape
    if tuple(k8.shape) != (B, H, N, d) or tuple(o.shape) != (B, H, N, d):
        raise KQError("k8 and o must match q8's shape")
    if v_layout == KQ_LAYOUT_TRANSPOSED and v8t.numel() != B * H * d * kq_vt_ld(N):
        raise KQError("v8t must be [B*H, d, kq_vt_ld(N)]")
    if row_stats is not None and row_stats.numel() != B * H * N * 2:
        raise KQError("row_stats must be [B, H, N, 2]")
    ws = _opt(workspace, torch.uint8, "workspace")
    nbytes = 0 if workspace is None else workspace.numel()
    _check(load().kq_attn_quant_fwd_ws(
        _dev(q8, torch.uint8, "q8"), _dev(k8, torch.uint8, "k8"), _dev(v8t, torch.uint8, "v8"),
        v_layout, B, H, N, d, float(s_q), float(s_k), float(s_v), float(sm_scale),
        _dev(o, torch.float32, "o"), _opt(row_stats, torch.float32, "row_stats"), ws, nbytes,
        _stream(stream)), "kq_attn_quant_fwd_ws")


def kq_attn_quant_fwd_qbf16(q, inv_scale_q: float, k8, v8t, s_q: float, s_k: float, s_v: float,
                            sm_scale: float, o, workspace, row_stats=None,
                            v_layout: int = KQ_LAYOUT_TRANSPOSED, stream=None):
    """kq_attn_quant_fwd_ws with Q in bf16 [B, H, N, 128], quantized inside the kernel with
    inv_scale_q (the codes kq_quantize_fp8_tensor forms; the result equals quantizing Q first,
    bit for bit)."""
    import torch
    B, H, N, d = q.shape
    if tuple(k8.shape) != (B, H, N, d) or tuple(o.shape) != (B, H, N, d):
        raise KQError("k8 and o must match q's shape")
    if v_layout == KQ_LAYOUT_TRANSPOSED and v8t.numel() != B * H * d * kq_vt_ld(N):
        raise KQError("v8t must be [B*H, d, kq_vt_ld(N)]")
    if row_stats is not None and row_stats.numel() != B * H * N * 2:
        raise KQError("row_stats must be [B, H, N, 2]")
    ws = _opt(workspace, torch.uint8, "workspace")
    nbytes = 0 if workspace is None else workspace.numel()
    _check(load().kq_attn_quant_fwd_qbf16(
        _dev(q, torch.bfloat16, "q"), float(inv_scale_q), _dev(k8, torch.uint8, "k8"),
        _dev(v8t, torch.uint8, "v8"), v_layout, B, H, N, d, float(s_q), float(s_k), float(s_v),
        float(sm_scale), _dev(o, torch.float32, "o"), _opt(row_stats, torch.float32, "row_stats"),
        ws, nbytes, _stream(stream)), "kq_attn_quant_fwd_qbf16")


def kq_attn_quant_fwd_noalloc(q8, k8, v8t, s_q: float, s_k: float, s_v: float, sm_scale: float,
                              o, row_stats=None, v_layout: int = KQ_LAYOUT_TRANSPOSED,
                              stream=None):
    """kq_attn_quant_fwd_ws with the key-split workspace in the library's static device array
    (no allocation anywhere: for callers that cannot allocate).  Arguments as
    kq_attn_quant_fwd; calls that overlap on one GPU race on the shared array."""
    import torch
    B, H, N, d = _attn_shapes(q8, k8, v8t, v_layout, o)
    if row_stats is not None and row_stats.numel() != B * H * N * 2:
        raise KQError("row_stats must be [B, H, N, 2]")
    _check(load().kq_attn_quant_fwd_noalloc(
        _dev(q8, torch.uint8, "q8"), _dev(k8, torch.uint8, "k8"), _dev(v8t, torch.uint8, "v8"),
        v_layout, B, H, N, d, float(s_q), float(s_k), float(s_v), float(sm_scale),
        _dev(o, torch.float32, "o"), _opt(row_stats, torch.float32, "row_stats"),
        _stream(stream)), "kq_attn_quant_fwd_noalloc")


def kq_attn_mxfp4_fwd(q_codes, q_scales, k_codes, k_scales, v8t, s_v: float, sm_scale: float,
                      o, workspace=None, row_stats=None, v_layout: int = KQ_LAYOUT_TRANSPOSED,
                      stream=None):
    """Attention with BMM1 on the FP4 block-quantized Q, K.  q_codes, k_codes: uint8
    [B, H, N, 64]; q_scales, k_scales: uint8 [B, H, N, 4]; v8t, o, row_stats as
    kq_attn_quant_fwd; workspace as kq_attn_quant_fwd_ws (or None)."""
    import torch
    B, H, N, dh = q_codes.shape
    d = 2 * dh
    if tuple(k_codes.shape) != (B, H, N, dh) or tuple(o.shape) != (B, H, N, d):
        raise KQError("k_codes and o must match q_codes' shape")
    if q_scales.numel() != B * H * N * (d // 32) or k_scales.numel() != B * H * N * (d // 32):
        raise KQError("scales must be [B, H, N, d/32]")
    if v_layout == KQ_LAYOUT_TRANSPOSED and v8t.numel() != B * H * d * kq_vt_ld(N):
        raise KQError("v8t must be [B*H, d, kq_vt_ld(N)]")
    if row_stats is not None and row_stats.numel() != B * H * N * 2:
        raise KQError("row_stats must be [B, H, N, 2]")
    ws = _opt(workspace, torch.uint8, "workspace")
    nbytes = 0 if workspace is None else workspace.numel()
    _check(load().kq_attn_mxfp4_fwd(
        _dev(q_codes, torch.uint8, "q_codes"), _dev(q_scales, torch.uint8, "q_scales"),
        _dev(k_codes, torch.uint8, "k_codes"), _dev(k_scales, torch.uint8, "k_scales"),
        _dev(v8t, torch.uint8, "v8"), v_layout, B, H, N, d, float(s_v), float(sm_scale),
        _dev(o, torch.float32, "o"), _opt(row_stats, torch.float32, "row_stats"), ws, nbytes,
        _stream(stream)), "kq_attn_mxfp4_fwd")


def _attn_shapes(q8, k8, v8t, v_layout, o=None):
    B, H, N, d = q8.shape
    if tuple(k8.shape) != (B, H, N, d) or (o is not None and tuple(o.shape) != (B, H, N, d)):
        raise KQError("k8 and o must match q8's shape")
    if v_layout == KQ_LAYOUT_TRANSPOSED and v8t.numel() != B * H * d * kq_vt_ld(N):
        raise KQError("v8t must be [B*H, d, kq_vt_ld(N)]")
    return B, H, N, d


def kq_attn_r1_stats(q8, k8, v8t, s_q: float, s_k: float, s_v: float, sm_scale: float,
                     row_stats4, workspace=None, v_layout: int = KQ_LAYOUT_TRANSPOSED,
                     stream=None):
    """First pass of R1: row_stats4 (float32 [B, H, N, 4]) = (M, l, max p, 0) per row;
    workspace as kq_attn_quant_fwd_ws (or None)."""
    import torch
    B, H, N, d = _attn_shapes(q8, k8, v8t, v_layout)
    if row_stats4.numel() != B * H * N * 4:
        raise KQError("row_stats4 must be [B, H, N, 4]")
    nbytes = 0 if workspace is None else workspace.numel()
    _check(load().kq_attn_r1_stats(
        _dev(q8, torch.uint8, "q8"), _dev(k8, torch.uint8, "k8"), _dev(v8t, torch.uint8, "v8"),
        v_layout, B, H, N, d, float(s_q), float(s_k), float(s_v), float(sm_scale),
        _dev(row_stats4, torch.float32, "row_stats4"),
        _opt(workspace, torch.uint8, "workspace"), nbytes, _stream(stream)), "kq_attn_r1_stats")


def kq_attn_r1_amax(row_stats4, amax, stream=None):
    """amax[0] = max(amax[0], largest normalized probability in row_stats4)."""
    import torch
    if row_stats4.numel() % 4 or amax.numel() != 1:
        raise KQError("row_stats4 must be [..., 4] and amax one float32")
    _check(load().kq_attn_r1_amax(_dev(row_stats4, torch.float32, "row_stats4"),
                                  row_stats4.numel() // 4, _dev(amax, torch.float32, "amax"),
                                  _stream(stream)), "kq_attn_r1_amax")


def kq_attn_r1_fwd(q8, k8, v8t, s_q: float, s_k: float, s_v: float, sm_scale: float,
                   amax_p: float, o, row_stats4, workspace=None,
                   v_layout: int = KQ_LAYOUT_TRANSPOSED, stream=None):
    """R1 attention (both passes) with the static amax_P; row_stats4 float32 [B, H, N, 4];
    workspace as kq_attn_quant_fwd_ws (or None)."""
    import torch
    B, H, N, d = _attn_shapes(q8, k8, v8t, v_layout, o)
    if row_stats4.numel() != B * H * N * 4:
        raise KQError("row_stats4 must be [B, H, N, 4]")
    _check(load().kq_attn_r1_fwd(
        _dev(q8, torch.uint8, "q8"), _dev(k8, torch.uint8, "k8"), _dev(v8t, torch.uint8, "v8"),
        v_layout, B, H, N, d, float(s_q), float(s_k), float(s_v), float(sm_scale),
        float(amax_p), _dev(o, torch.float32, "o"),
        _dev(row_stats4, torch.float32, "row_stats4"), _opt(workspace, torch.uint8, "workspace"),
        0 if workspace is None else workspace.numel(), _stream(stream)), "kq_attn_r1_fwd")


def _gemm_fp8(a8, b8, s_a, s_b, c, out_bf16, stream):
    import torch
    M, K = a8.shape
    N = b8.shape[0]
    if b8.dim() != 2 or b8.shape[1] != K or tuple(c.shape) != (M, N):
        raise KQError("expected a8 [M, K], b8 [N, K], c [M, N]")
    fn = "kq_gemm_fp8_bf16" if out_bf16 else "kq_gemm_fp8"
    _check(getattr(load(), fn)(
        _dev(a8, torch.uint8, "a8"), _dev(b8, torch.uint8, "b8"), M, N, K, float(s_a),
        float(s_b), _dev(c, torch.bfloat16 if out_bf16 else torch.float32, "c"),
        _stream(stream)), fn)


def kq_gemm_fp8(a8, b8, s_a: float, s_b: float, c, stream=None):
    """C = s_a s_b E4M3(a8) E4M3(b8)^T.  a8: uint8 [M, K]; b8: uint8 [N, K]; c: float32 [M, N]."""
    _gemm_fp8(a8, b8, s_a, s_b, c, False, stream)


def kq_gemm_fp8_bf16(a8, b8, s_a: float, s_b: float, c, stream=None):
    """kq_gemm_fp8 with c bf16 [M, N]: each value the float32 result rounded once (RNE)."""
    _gemm_fp8(a8, b8, s_a, s_b, c, True, stream)


def _gemm_mxfp4(a_codes, a_scales, b_codes, b_scales, c, out_bf16, stream):
    import torch
    M, Kh = a_codes.shape
    N = b_codes.shape[0]
    K = 2 * Kh
    if (b_codes.dim() != 2 or b_codes.shape[1] != Kh or a_scales.numel() != M * (K // 32)
            or b_scales.numel() != N * (K // 32) or tuple(c.shape) != (M, N)):
        raise KQError("expected codes [rows, K/2], scales [rows, K/32], c [M, N]")
    fn = "kq_gemm_mxfp4_bf16" if out_bf16 else "kq_gemm_mxfp4"
    _check(getattr(load(), fn)(
        _dev(a_codes, torch.uint8, "a_codes"), _dev(a_scales, torch.uint8, "a_scales"),
        _dev(b_codes, torch.uint8, "b_codes"), _dev(b_scales, torch.uint8, "b_scales"),
        M, N, K, _dev(c, torch.bfloat16 if out_bf16 else torch.float32, "c"),
        _stream(stream)), fn)


def kq_gemm_mxfp4(a_codes, a_scales, b_codes, b_scales, c, stream=None):
    """C = dq(a) dq(b)^T from packed E2M1 codes [rows, K/2] and E8M0 scales [rows, K/32];
    c: float32 [M, N]."""
    _gemm_mxfp4(a_codes, a_scales, b_codes, b_scales, c, False, stream)


def kq_gemm_mxfp4_bf16(a_codes, a_scales, b_codes, b_scales, c, stream=None):
    """kq_gemm_mxfp4 with c bf16 [M, N]: each value the float32 result rounded once (RNE)."""
    _gemm_mxfp4(a_codes, a_scales, b_codes, b_scales, c, True, stream)


def kq_svdquant_down(a, l_down, t, stream=None):
    """T = bf16(A L_down^T) for the SVD-Quant branch: a bf16 [M, K], l_down bf16 [r, K],
    t bf16 [M, r]."""
    import torch
    M, K = a.shape
    r = l_down.shape[0]
    if l_down.dim() != 2 or l_down.shape[1] != K or tuple(t.shape) != (M, r):
        raise KQError("expected a [M, K], l_down [r, K], t [M, r]")
    _check(load().kq_svdquant_down(_dev(a, torch.bfloat16, "a"),
                                   _dev(l_down, torch.bfloat16, "l_down"), M, K, r,
                                   _dev(t, torch.bfloat16, "t"), _stream(stream)),
           "kq_svdquant_down")


def _gemm_svdquant(a_codes, a_scales, r_codes, r_scales, t, l_up, c, out_bf16, stream):
    import torch
    M, Kh = a_codes.shape
    N = r_codes.shape[0]
    K = 2 * Kh
    rank = t.shape[1]
    if (r_codes.dim() != 2 or r_codes.shape[1] != Kh or a_scales.numel() != M * (K // 32)
            or r_scales.numel() != N * (K // 32) or tuple(c.shape) != (M, N)
            or tuple(t.shape) != (M, rank) or tuple(l_up.shape) != (N, rank)):
        raise KQError("expected codes [rows, K/2], scales [rows, K/32], t [M, r], l_up [N, r], "
                      "c [M, N]")
    fn = "kq_gemm_mxfp4_svdquant_bf16" if out_bf16 else "kq_gemm_mxfp4_svdquant"
    _check(getattr(load(), fn)(
        _dev(a_codes, torch.uint8, "a_codes"), _dev(a_scales, torch.uint8, "a_scales"),
        _dev(r_codes, torch.uint8, "r_codes"), _dev(r_scales, torch.uint8, "r_scales"),
        M, N, K, _dev(t, torch.bfloat16, "t"), _dev(l_up, torch.bfloat16, "l_up"), rank,
        _dev(c, torch.bfloat16 if out_bf16 else torch.float32, "c"), _stream(stream)), fn)


def kq_gemm_mxfp4_svdquant(a_codes, a_scales, r_codes, r_scales, t, l_up, c, stream=None):
    """C = dq(a) dq(r)^T + t l_up^T: the MXFP4 GEMM of the activations and the SVD-Quant
    residual plus the bf16 branch; c float32 [M, N]."""
    _gemm_svdquant(a_codes, a_scales, r_codes, r_scales, t, l_up, c, False, stream)


def kq_gemm_mxfp4_svdquant_bf16(a_codes, a_scales, r_codes, r_scales, t, l_up, c, stream=None):
    """kq_gemm_mxfp4_svdquant with c bf16 [M, N]: each value the float32 result rounded once."""
    _gemm_svdquant(a_codes, a_scales, r_codes, r_scales, t, l_up, c, True, stream)


def kq_svdquant_factorize(w_bits, rank: int):
    """Offline SVD-Quant weight step (host C code): from bf16 weights given as bit patterns
    (numpy uint16 [N, K]), returns (l_up [N, r], l_down [r, K], residual [N, K]) as bf16 bit
    patterns (numpy uint16)."""
    w = np.ascontiguousarray(w_bits, dtype=np.uint16)
    if w.ndim != 2:
        raise KQError("w must be [N, K]")
    N, K = w.shape
    l_up = np.empty((N, rank), np.uint16)
    l_down = np.empty((rank, K), np.uint16)
    res = np.empty((N, K), np.uint16)
    _check(load().kq_svdquant_factorize(w.ctypes.data_as(_P), N, K, int(rank),
                                        l_up.ctypes.data_as(_P), l_down.ctypes.data_as(_P),
                                        res.ctypes.data_as(_P)), "kq_svdquant_factorize")
    return l_up, l_down, res


def kq_svdquant_activations(a, l_down, codes, scales, t, stream=None):
    """One pass over the activations a (bf16 [M, K]): their MXFP4 codes (uint8 [M, K/2]) and
    E8M0 scales (uint8 [M, K/32]), as kq_quantize_fp4_block, and T = bf16(a l_down^T)
    (t bf16 [M, r], l_down bf16 [r, K])."""
    import torch
    M, K = a.shape
    r = l_down.shape[0]
    if (l_down.dim() != 2 or l_down.shape[1] != K or tuple(t.shape) != (M, r)
            or codes.numel() != M * K // 2 or scales.numel() != M * K // 32):
        raise KQError("expected a [M, K], l_down [r, K], codes [M, K/2], scales [M, K/32], "
                      "t [M, r]")
    _check(load().kq_svdquant_activations(
        _dev(a, torch.bfloat16, "a"), _dev(l_down, torch.bfloat16, "l_down"), M, K, r,
        _dev(codes, torch.uint8, "codes"), _dev(scales, torch.uint8, "scales"),
        _dev(t, torch.bfloat16, "t"), _stream(stream)), "kq_svdquant_activations")
