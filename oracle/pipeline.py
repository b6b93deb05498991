"""The whole quantized SDPA path for one workload, step by step.

Order of the steps (NVIDIA blog "Optimizing FLUX.1 Kontext for Image Editing with
Low-Precision Quantization", section "Workflow and Quantization" and Fig. 4;
positions from lpnh.cn "Flux.1 Kontext deep dive", sections 1 and 3):

  1. [RoPE workloads] rotate Q and K with the 3-axis rotary embedding (float32);
  2. [FP4 workloads] per-block FP4 fake-quant of Q, K and V (quantize, dequantize);
  3. calibrate each tensor's amax on the input of its FP8 quantizer (static scale);
  4. per-tensor FP8 quantization of Q, K and V (BMM1 / BMM2 inputs);
  5. R3 attention: BMM1 in FP8 with FP32 accumulation, FP32 softmax, FP8 P, BMM2.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

from . import attention as A
from . import formats as F
from . import quant as Qz
from . import rope as R


@dataclasses.dataclass
class Quantized:
    """Everything the path produces up to the attention inputs."""
    x: dict            # float32 input of the FP8 quantizer per tensor name
    fp4: dict          # name -> (codes, scales, dq) for FP4 workloads
    amax: dict         # name -> float
    scale: dict        # name -> (s, inv) float32
    codes: dict        # name -> uint8 E4M3 codes [B, H, N, d]
    rope_table: Optional[np.ndarray] = None


def quantize_inputs(q_bits, k_bits, v_bits, mode: str = "fp8", positions=None) -> Quantized:
    """Steps 1-4 for bf16 inputs given as bit arrays [B, H, N, d]."""
    x = {"q": F.bf16_bits_to_f32(q_bits), "k": F.bf16_bits_to_f32(k_bits),
         "v": F.bf16_bits_to_f32(v_bits)}
    tab = None
    if positions is not None:
        tab = R.table(positions)
        x["q"] = R.apply(x["q"], tab)
        x["k"] = R.apply(x["k"], tab)
    fp4 = {}
    if mode == "fp4":
        for n in ("q", "k", "v"):
            fp4[n] = Qz.fp4_block_quant(x[n])
            x[n] = fp4[n][2]
    elif mode != "fp8":
        raise ValueError(mode)
    amax = {n: Qz.amax(x[n]) for n in x}
    scale = {n: Qz.fp8_scales(amax[n]) for n in x}
    codes = {n: Qz.fp8_codes(x[n], scale[n][1]) for n in x}
    return Quantized(x=x, fp4=fp4, amax=amax, scale=scale, codes=codes, rope_table=tab)


def attention(qz: Quantized, rows=None, sm_scale=None):
    """Step 5 on the quantized inputs; returns (O, M, l) for the requested query rows."""
    d = qz.codes["q"].shape[-1]
    if sm_scale is None:
        sm_scale = np.float32(1.0 / math.sqrt(d))
    return A.attention_r3(qz.codes["q"], qz.codes["k"], qz.codes["v"], qz.scale["q"][0],
                          qz.scale["k"][0], qz.scale["v"][0], sm_scale, rows=rows)
