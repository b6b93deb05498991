"""The quantized SDPA path as a sequence of libkq calls on device tensors.

Order of the steps (NVIDIA blog "Optimizing FLUX.1 Kontext for Image Editing with
Low-Precision Quantization", section "Workflow and Quantization" and Fig. 4):

  offline, once (workflow step 4, post-training calibration with static scales):
    [RoPE] -> [FP4 block fake-quant] -> amax of each FP8 quantizer's input -> (s, 1/s)
  every forward:
    Q, K: [RoPE] -> [FP4 block quant] -> per-tensor FP8          (one fused kernel each)
    V:    [FP4 block quant] -> per-tensor FP8, transposed layout
    fused attention: FP8 BMM1, FP32 softmax, FP8 P, FP8 BMM2
  (FP8 mode, one-pass P: Q's per-tensor FP8 step runs inside the attention kernel, on its one
  read of Q, with the quantizer's codes.)

Every step runs in libkq's kernels; this module only allocates outputs and passes
pointers.  Calibration copies one float per tensor to the host to derive the static scales.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

from . import (KQ_LAYOUT_TRANSPOSED, KQError, kq_amax_calibrate, kq_attn_mxfp4_fwd,
               kq_attn_quant_fwd_qbf16, kq_attn_quant_fwd_ws,
               kq_attn_r1_amax, kq_attn_r1_fwd, kq_attn_r1_stats,
               kq_attn_workspace_size,
               kq_fp8_scales_from_amax, kq_quantize_fp4_block, kq_quantize_fp8_tensor,
               kq_rope3_table, kq_vt_ld)


@dataclasses.dataclass
class Buffers:
    q8: torch.Tensor
    k8: torch.Tensor
    v8t: torch.Tensor
    o: torch.Tensor
    stats: Optional[torch.Tensor]
    fp4: dict                 # name -> (codes, scales)
    v_dq: Optional[torch.Tensor]


class QuantizedSDPA:
    """Quantized attention for inputs of shape [B, H, N, 128] in bf16.

    mode "fp8": per-tensor FP8 Q/K/V.  mode "fp4": per-block FP4 Q/K/V, then per-tensor FP8.
    positions: optional int32 [N, 3] token positions; enables the 3-axis rotary embedding of
    Q and K before FP4 quantization (FP4 mode only).
    native_fp4 (FP4 mode only): BMM1 multiplies the FP4 Q, K directly (E2M1 + E8M0 on the
    matrix cores) instead of their per-tensor FP8 re-quantization; V still goes FP4 -> FP8.
    p_reading "r3" (default): the one-pass reading (static 1/448 scale on exp2(t - M), row sum
    after BMM2).  "r1": the literal FakeQuantize of the normalized P with a calibrated
    per-tensor amax_P, two passes (FP8 BMM1 only).
    fuse_q (FP8 mode, "r3" only; default on there): forward() quantizes Q inside the attention
    kernel (kq_attn_quant_fwd_qbf16, bit-identical codes and output) and leaves buf.q8
    unwritten; quantize() still writes all three FP8 tensors.
    """

    def __init__(self, B, H, N, d=128, mode="fp8", positions=None, device="cuda",
                 sm_scale=None, want_stats=False, native_fp4=False, p_reading="r3",
                 fuse_q=None):
        if mode not in ("fp8", "fp4"):
            raise ValueError(mode)
        if native_fp4 and mode != "fp4":
            raise ValueError("native_fp4 needs mode 'fp4'")
        self.native_fp4 = native_fp4
        if p_reading not in ("r3", "r1") or (p_reading == "r1" and native_fp4):
            raise ValueError(p_reading)
        self.p_reading = p_reading
        self.amax_p = None
        can_fuse = mode == "fp8" and p_reading == "r3"
        if fuse_q and not can_fuse:
            raise ValueError("fuse_q needs mode 'fp8' and p_reading 'r3'")
        self.fuse_q = can_fuse if fuse_q is None else bool(fuse_q)
        self._q_bf16 = None           # Q of the prepared forward when fuse_q
        if positions is not None and mode != "fp4":
            raise ValueError("the rotary embedding is fused into the FP4 quantizer")
        self.B, self.H, self.N, self.d, self.mode = B, H, N, d, mode
        self.device = torch.device(device)
        self.sm_scale = float(np.float32(1.0 / math.sqrt(d))) if sm_scale is None else sm_scale
        self.rope = None
        if positions is not None:
            table = torch.from_numpy(kq_rope3_table(positions)).to(self.device)
            self.rope = (table, N)
        self.scales = None            # name -> (s, inv), static after calibrate()
        self.workspace = None         # attention workspace (allocated on first use)
        self.amax = None
        shape = (B, H, N, d)
        u8 = dict(dtype=torch.uint8, device=self.device)
        fp4 = {}
        if mode == "fp4":
            for n in "qkv":
                fp4[n] = (torch.empty((B, H, N, d // 2), **u8), torch.empty((B, H, N, d // 32), **u8))
        self.buf = Buffers(
            q8=torch.empty(shape, **u8), k8=torch.empty(shape, **u8),
            v8t=torch.empty((B * H, d, kq_vt_ld(N)), **u8),
            o=torch.empty(shape, dtype=torch.float32, device=self.device),
            stats=torch.empty((B, H, N, 2), dtype=torch.float32, device=self.device)
            if want_stats else None,
            fp4=fp4,
            v_dq=torch.empty(shape, dtype=torch.bfloat16, device=self.device)
            if mode == "fp4" else None)

    def _rope_for(self, name):
        return self.rope if (self.rope is not None and name in "qk") else None

    def calibrate(self, q, k, v):
        """Static per-tensor scales from max calibration over (q, k, v) (offline step)."""
        amax = torch.zeros(3, dtype=torch.float32, device=self.device)
        for i, (n, x) in enumerate(zip("qkv", (q, k, v))):
            src = x
            if self.mode == "fp4":
                dq = torch.empty_like(x)
                codes, scales = self.buf.fp4[n]
                kq_quantize_fp4_block(x, codes, scales, dq=dq, rope=self._rope_for(n))
                src = dq
            kq_amax_calibrate(src, amax[i:i + 1])
        a = amax.cpu().numpy()
        self.amax = {n: float(a[i]) for i, n in enumerate("qkv")}
        self.scales = {n: kq_fp8_scales_from_amax(a[i]) for i, n in enumerate("qkv")}
        if self.native_fp4:
            # the MXFP4 BMM1 needs |t| < 2^20: |raw| <= 128 max|dq(q)| max|dq(k)|
            bound = self.sm_scale * math.log2(math.e) * 128.0 * self.amax["q"] * self.amax["k"]
            if not bound < 2.0 ** 20:
                raise KQError(f"native MXFP4 BMM1: scores may reach {bound:.3g} in the exp2 "
                              "domain (limit 2^20); use the FP8 BMM1 (native_fp4=False)")
        if self.p_reading == "r1":
            # amax_P: the largest normalized probability over the calibration inputs
            self.quantize(q, k, v)
            b = self.buf
            st = self._r1_stats()
            kq_attn_r1_stats(b.q8, b.k8, b.v8t, self.scales["q"][0], self.scales["k"][0],
                             self.scales["v"][0], self.sm_scale, st, self._workspace())
            am = torch.zeros(1, dtype=torch.float32, device=self.device)
            kq_attn_r1_amax(st, am)
            self.amax_p = float(am.item())
        return self.scales

    def _r1_stats(self):
        if getattr(self, "_st4", None) is None:
            self._st4 = torch.empty((self.B, self.H, self.N, 4), dtype=torch.float32,
                                    device=self.device)
        return self._st4

    def prepare(self, q, k, v):
        """The per-forward quantization that precedes attention(): with fuse_q, K and V only
        (Q is quantized inside the attention kernel); otherwise quantize()."""
        if not self.fuse_q:
            self.quantize(q, k, v)
            return
        b = self.buf
        kq_quantize_fp8_tensor(k, self.scales["k"][1], b.k8)
        kq_quantize_fp8_tensor(v, self.scales["v"][1], b.v8t, layout=KQ_LAYOUT_TRANSPOSED)
        self._q_bf16 = q

    def quantize(self, q, k, v):
        """Per-forward quantization of Q, K, V into the FP8 attention inputs (all three, into
        buf; attention() then reads Q's codes from buf.q8)."""
        self._q_bf16 = None
        b = self.buf
        if self.mode == "fp8":
            kq_quantize_fp8_tensor(q, self.scales["q"][1], b.q8)
            kq_quantize_fp8_tensor(k, self.scales["k"][1], b.k8)
            kq_quantize_fp8_tensor(v, self.scales["v"][1], b.v8t, layout=KQ_LAYOUT_TRANSPOSED)
        elif self.native_fp4:
            for n, x in (("q", q), ("k", k)):
                codes, scales = b.fp4[n]
                kq_quantize_fp4_block(x, codes, scales, rope=self._rope_for(n))
            codes, scales = b.fp4["v"]
            kq_quantize_fp4_block(v, codes, scales, dq=b.v_dq)
            kq_quantize_fp8_tensor(b.v_dq, self.scales["v"][1], b.v8t, layout=KQ_LAYOUT_TRANSPOSED)
        else:
            for n, x, out in (("q", q, b.q8), ("k", k, b.k8)):
                codes, scales = b.fp4[n]
                kq_quantize_fp4_block(x, codes, scales, fp8=out, inv_scale8=self.scales[n][1],
                                      rope=self._rope_for(n))
            codes, scales = b.fp4["v"]
            kq_quantize_fp4_block(v, codes, scales, dq=b.v_dq)
            kq_quantize_fp8_tensor(b.v_dq, self.scales["v"][1], b.v8t, layout=KQ_LAYOUT_TRANSPOSED)

    def _workspace(self):
        if self.workspace is None:
            nbytes = kq_attn_workspace_size(self.B, self.H, self.N, self.d)
            self.workspace = (torch.empty(nbytes, dtype=torch.uint8, device=self.device)
                              if nbytes else False)
        return self.workspace if self.workspace is not False else None

    def attention(self):
        b = self.buf
        ws = self._workspace()
        if self.p_reading == "r1":
            kq_attn_r1_fwd(b.q8, b.k8, b.v8t, self.scales["q"][0], self.scales["k"][0],
                           self.scales["v"][0], self.sm_scale, self.amax_p, b.o,
                           self._r1_stats(), ws)
        elif self.native_fp4:
            (qc, qs), (kc, ks) = b.fp4["q"], b.fp4["k"]
            kq_attn_mxfp4_fwd(qc, qs, kc, ks, b.v8t, self.scales["v"][0], self.sm_scale, b.o,
                              ws, row_stats=b.stats)
        elif self._q_bf16 is not None:
            kq_attn_quant_fwd_qbf16(self._q_bf16, self.scales["q"][1], b.k8, b.v8t,
                                    self.scales["q"][0], self.scales["k"][0], self.scales["v"][0],
                                    self.sm_scale, b.o, ws, row_stats=b.stats)
        else:
            kq_attn_quant_fwd_ws(b.q8, b.k8, b.v8t, self.scales["q"][0], self.scales["k"][0],
                                 self.scales["v"][0], self.sm_scale, b.o, ws, row_stats=b.stats)
        return b.o

    def forward(self, q, k, v):
        self.prepare(q, k, v)
        return self.attention()


def bf16_from_bits(bits: np.ndarray, device="cuda") -> torch.Tensor:
    """Device bf16 tensor holding the given bf16 bit patterns (uint16 numpy array)."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.to(device)
