"""CPU oracle for quantized scaled-dot-product attention — TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct numpy implementation of what the quantized
attention path computes, written from the method's description:

  NVIDIA Technical Blog, "Optimizing FLUX.1 Kontext for Image Editing with
  Low-Precision Quantization", section "Workflow and Quantization" (the four-part
  SDPA quantization strategy and Fig. 4): Q/K/V quantized per-tensor FP8 or
  per-block FP4; BMM1 (QK^T) on FP8 inputs with higher-precision accumulation;
  softmax in FP32 without quantization; BMM2 (P.V) with per-tensor FP8; the
  "Quant" nodes are FakeQuantize (quantize then dequantize) operations.

Number formats follow their public definitions: the OCP 8-bit floating point
specification (E4M3, "FN" flavour: bias 7, max 448, no infinities) and the OCP
Microscaling (MX) specification v1.0 (E2M1 elements, E8M0 shared scales).

Only `tests/`, `__graft_entry__.smoke()` and `bench.py`'s CPU-baseline leg may
import this package.  The HIP library never does, and this package shares no
code with it; both take their inputs from the separate `workloads` module.

Modules:
  formats    E4M3 / E2M1 / E8M0 encode and decode by nearest-value search
  quant      amax, per-tensor FP8 scale rule, FP8 fake-quant, FP4 block fake-quant
  rope       3-axis rotary position embedding (table and rotation)
  attention  R3 quantized attention (gated), R1 variant and FP64 reference (reported)
  pipeline   the whole path for one workload: RoPE -> FP4 -> calibrate -> FP8 -> attention
  gemm       quantized projection GEMMs (per-tensor FP8 W8A8, per-block MXFP4), exact float64
  svdquant   SVD-Quant in FP4 of a projection GEMM: rank-r bf16 branch + MXFP4 residual
"""
