"""Benchmark of the quantized SDPA hot path on one MI355X.

Workload: FLUX.1 Kontext 1024x1024 edit, B=1, H=24, N=8704 (512 text + 4096 target + 4096
context tokens), d=128, per-tensor FP8 Q/K/V/P, FP32 softmax (seeded synthetic bf16 inputs
~N(0,1) with 1% outlier channels x20).  One step = one pass of the per-forward path:
FP8 quantization of Q, K, V (static scales from an offline max calibration done before the
timed region) followed by the fused attention kernel.

Prints ONE JSON line.  `value` = attention FLOPs (4*B*H*N^2*d) per step / step time, in
TFLOP/s.  `roofline` describes the attention kernel alone, timed with HIP events on the
stream it runs on, around its launch in each timed step.  `cpu_baseline` times the CPU oracle on a bounded sample of the same
workload (a subset of query rows of a few heads).

`--gemm fp8|mxfp4 --gemm-shape qkv|out` instead times one quantized projection GEMM around the
attention (C = A W^T with A the 8704 token activations, K = 3072; N = 9216 for the QKV
projection, 3072 for the output projection): codes and scales are prepared before the timed
region, a step is one GEMM launch, and the line's cpu_baseline is the exact oracle GEMM on a
bounded sample of activation rows.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

FP8_PEAK_TFLOPS = 5000.0      # MI355X dense FP8 MFMA peak
FP4_PEAK_TFLOPS = 10100.0     # MI355X dense FP4 MFMA peak
HBM_PEAK_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # ~0.1 s of untimed steps: the clock under this load needs about that long to settle
    ap.add_argument("--warmup", type=int, default=150)
    ap.add_argument("--config", type=int, default=3, help="workload number (1-5)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=20.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--heads", type=int, default=None,
                    help="override the workload's head count, e.g. 3 = one GPU's share of the "
                         "Kontext heads under 8-way head sharding")
    ap.add_argument("--native-fp4", action="store_true",
                    help="FP4 workloads: BMM1 on the FP4 Q, K (E2M1 + E8M0) instead of their "
                         "FP8 re-quantization")
    ap.add_argument("--p-reading", choices=["r3", "r1"], default="r3",
                    help="r1: the literal FakeQuantize of the normalized P, two passes, with "
                         "amax_P calibrated offline")
    ap.add_argument("--gemm", choices=["fp8", "mxfp4"], default=None,
                    help="time a projection GEMM instead of the attention step")
    ap.add_argument("--gemm-shape", choices=["qkv", "out"], default="qkv")
    ap.add_argument("--gemm-out", choices=["f32", "bf16"], default="f32",
                    help="C in float32 (kq_gemm_*) or bf16 (kq_gemm_*_bf16)")
    ap.add_argument("--pmc-workload", action="store_true",
                    help="no timing: a plain copy of COPY_BYTES (counter calibration), then 3 "
                         "steps; run under rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE")
    return ap.parse_args()


COPY_BYTES = 1 << 30          # calibration copy for the HBM byte counters
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_fp8_kontext1024_traffic.txt")
KERNEL_SRC = os.path.join(ROOT, "precision_quantized_attention_amd", "csrc", "attn_fp8.hip")


def kernel_sha() -> str:
    import hashlib
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic_bytes():
    """HBM bytes per attention launch from the committed counter summary, or None when the
    summary is missing or was taken on a different kernel source."""
    try:
        fields = {}
        with open(TRAFFIC_FILE) as f:
            for line in f:
                if ":" in line and not line.startswith("#"):
                    k, v = line.split(":", 1)
                    fields[k.strip()] = v.strip()
        if fields.get("kernel_sha") != kernel_sha():
            return None
        return int(float(fields["attn_fetch_bytes_per_launch"]) +
                   float(fields["attn_write_bytes_per_launch"]))
    except (OSError, KeyError, ValueError):
        return None


def host_cpu() -> str:
    """Model name of the host CPU the oracle baseline runs on (Linux /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg, target_s):
    """Time the CPU oracle (as it stands) on a bounded sample of the workload: the full
    per-tensor quantization of Q, K, V, then R3 attention for query rows of successive heads
    until about `target_s` seconds have been spent."""
    import numpy as np
    import torch
    import workloads as W
    from oracle import attention as A
    from oracle import pipeline as OP

    c = W.config(cfg)
    pos = W.positions(c) if c.rope else None
    t0 = time.perf_counter()
    qz = OP.quantize_inputs(*W.qkv_bits(cfg), mode=c.mode, positions=pos)
    t_quant = time.perf_counter() - t0
    rows_done, heads_done, t_attn = 0, 0, 0.0
    sm = np.float32(1 / math.sqrt(c.d))
    for b in range(c.B):
        for h in range(c.H):
            if t_attn + t_quant >= target_s:
                break
            sl = (slice(b, b + 1), slice(h, h + 1))
            for r0 in range(0, c.N, 1024):
                if t_attn + t_quant >= target_s:
                    break
                rows = np.arange(r0, min(c.N, r0 + 1024))
                t0 = time.perf_counter()
                A.attention_r3(qz.codes["q"][sl], qz.codes["k"][sl], qz.codes["v"][sl],
                               qz.scale["q"][0], qz.scale["k"][0], qz.scale["v"][0], sm,
                               rows=rows)
                t_attn += time.perf_counter() - t0
                rows_done += len(rows)
            heads_done += 1
    # attention FLOPs of the processed rows (4*N*d each) per second; the quantization of the
    # whole tensors is charged in proportion to the rows processed
    total_rows = c.B * c.H * c.N
    flops = 4.0 * rows_done * c.N * c.d
    t = t_attn + t_quant * rows_done / total_rows
    return {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": torch.get_num_threads(),
            "kind": "oracle",
            "sample": f"{c.name}: FP8 quantization of the full Q, K, V ({t_quant:.1f} s) and R3 "
                      f"attention for {rows_done} query rows in {heads_done} heads "
                      f"({t_attn:.1f} s); quantization charged pro rata"}


def gemm_main(args):
    """One JSON line for a projection GEMM: a step is one kq_gemm_* launch on codes prepared
    (quantized by the library's own kernels) before the timed region."""
    import numpy as np
    import torch
    import workloads as W
    import precision_quantized_attention_amd as kq
    from precision_quantized_attention_amd.pipeline import bf16_from_bits

    shape = W.GEMM_SHAPES[0 if args.gemm_shape == "qkv" else 1]
    M, N, K = shape.M, shape.N, shape.K
    torch.cuda.set_device(0)
    seed = 100 + N
    a_bits, w_bits = W.gemm_bits(M, N, K, seed)
    a, w = bf16_from_bits(a_bits), bf16_from_bits(w_bits)
    bf16_out = args.gemm_out == "bf16"
    c = torch.empty((M, N), dtype=torch.bfloat16 if bf16_out else torch.float32, device="cuda")
    if args.gemm == "fp8":
        ops = []
        for x in (a, w):
            am = torch.zeros(1, dtype=torch.float32, device="cuda")
            kq.kq_amax_calibrate(x, am)
            s_x, inv = kq.kq_fp8_scales_from_amax(float(am.item()))
            y = torch.empty(x.shape, dtype=torch.uint8, device="cuda")
            kq.kq_quantize_fp8_tensor(x, inv, y)
            ops.append((y, s_x))
        (a8, sa), (w8, sw) = ops
        gemm = kq.kq_gemm_fp8_bf16 if bf16_out else kq.kq_gemm_fp8
        launch = lambda: gemm(a8, w8, sa, sw, c)
        peak = FP8_PEAK_TFLOPS
    else:
        ops = []
        for x in (a, w):
            rows = x.shape[0]
            codes = torch.empty((rows, K // 2), dtype=torch.uint8, device="cuda")
            scales = torch.empty((rows, K // 32), dtype=torch.uint8, device="cuda")
            kq.kq_quantize_fp4_block(x.view(-1, 128), codes.view(-1, 64), scales.view(-1, 4))
            ops.append((codes, scales))
        (ac, asc), (wc, wsc) = ops
        gemm = kq.kq_gemm_mxfp4_bf16 if bf16_out else kq.kq_gemm_mxfp4
        launch = lambda: gemm(ac, asc, wc, wsc, c)
        peak = FP4_PEAK_TFLOPS
    stream = torch.cuda.current_stream()
    if args.pmc_workload:
        src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        for _ in range(3):
            launch()
        torch.cuda.synchronize()
        print(json.dumps({"pmc_workload": shape.name, "copy_bytes": COPY_BYTES, "steps": 3}))
        return
    for _ in range(args.warmup):
        launch()
    torch.cuda.synchronize()
    # timed steps; HIP events on the launch stream bracket each launch inside the timed region
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    t0 = time.perf_counter()
    for e0, e1 in ev:
        e0.record(stream)
        launch()
        e1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) / args.steps * 1e3
    kern_ms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in ev]))
    value = shape.flops / (ms_per_step * 1e-3) / 1e12
    achieved = shape.flops / (kern_ms * 1e-3) / 1e12
    fmt_name = "FP8 E4M3 per-tensor (W8A8)" if args.gemm == "fp8" else "MXFP4 (E2M1, E8M0 per 32)"
    out = {
        "metric": f"quantized projection GEMM TFLOP/s ({fmt_name})",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8_e4m3" if args.gemm == "fp8" else "mxfp4_e2m1", "data": "synthetic",
        "config": {"workload": shape.name, "M": M, "N": N, "K": K,
                   "step": "one GEMM launch on prepared codes, "
                           + ("bf16 C" if bf16_out else "float32 C")},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": None},
        "gemm_ms": round(kern_ms, 4),
    }
    if not args.no_cpu_baseline:
        out["host_cpu"] = host_cpu()
        out["cpu_baseline"] = gemm_cpu_baseline(args.gemm, shape, a_bits, w_bits,
                                                args.cpu_seconds)
    print(json.dumps(out))


def gemm_cpu_baseline(fmt, shape, a_bits, w_bits, target_s):
    """The oracle GEMM (exact float64) on successive 64-row blocks of the activations against
    all weights, quantized by the oracle, until about `target_s` seconds."""
    import numpy as np
    import torch
    import workloads as W
    from oracle import gemm as OG
    from oracle import quant as Qz

    t0 = time.perf_counter()
    wf = W.bits_to_f32(w_bits)
    if fmt == "fp8":
        sw, iw = Qz.fp8_scales(Qz.amax(wf))
        sa, ia = Qz.fp8_scales(Qz.amax(W.bits_to_f32(a_bits)))
        wq = Qz.fp8_codes(wf, iw)
    else:
        wq = Qz.fp4_block_quant(wf)[:2]
    t_w = time.perf_counter() - t0
    rows, t = 0, 0.0
    while t + t_w < target_s and rows < shape.M:
        af = W.bits_to_f32(a_bits[rows:rows + 64])
        t0 = time.perf_counter()
        if fmt == "fp8":
            OG.gemm_fp8(Qz.fp8_codes(af, ia), wq, sa, sw)
        else:
            ac, asc, _ = Qz.fp4_block_quant(af)
            OG.gemm_mxfp4(ac, asc, *wq)
        t += time.perf_counter() - t0
        rows += len(af)
    flops = 2.0 * rows * shape.N * shape.K
    return {"value": flops / (t + t_w * rows / shape.M) / 1e12, "unit": "TFLOP/s",
            "cores": torch.get_num_threads(), "kind": "oracle",
            "sample": f"{shape.name}: oracle quantization of the weights ({t_w:.1f} s, charged "
                      f"pro rata) and the exact GEMM of {rows} activation rows ({t:.1f} s)"}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build measures one GPU; --gpus must be 1"}))
        sys.exit(2)
    if args.gemm:
        gemm_main(args)
        return
    import numpy as np
    import torch
    import workloads as W
    from precision_quantized_attention_amd.pipeline import QuantizedSDPA, bf16_from_bits

    c = W.config(args.config)
    torch.cuda.set_device(0)
    q, k, v = (bf16_from_bits(b) for b in W.qkv_bits(args.config))
    if args.heads is not None:
        if not 1 <= args.heads <= c.H:
            print(json.dumps({"error": f"--heads must be in 1..{c.H}"}))
            sys.exit(2)
        import dataclasses
        q, k, v = (x[:, :args.heads].contiguous() for x in (q, k, v))
        c = dataclasses.replace(c, H=args.heads, name=f"{c.name}_h{args.heads}")
    if args.native_fp4 and c.mode != "fp4":
        print(json.dumps({"error": "--native-fp4 needs an FP4 workload (--config 4 or 5)"}))
        sys.exit(2)
    m = QuantizedSDPA(c.B, c.H, c.N, c.d, mode=c.mode,
                      positions=W.positions(c) if c.rope else None, native_fp4=args.native_fp4,
                      p_reading=args.p_reading)
    m.calibrate(q, k, v)                     # offline static calibration, not timed
    stream = torch.cuda.current_stream()

    if args.pmc_workload:
        src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        for _ in range(3):
            m.forward(q, k, v)
        torch.cuda.synchronize()
        print(json.dumps({"pmc_workload": c.name, "copy_bytes": COPY_BYTES, "steps": 3}))
        return

    for _ in range(args.warmup):
        m.forward(q, k, v)
    torch.cuda.synchronize()

    # timed steps (forward = quantize, then attention); HIP events on the attention's stream
    # bracket its launch inside each timed step
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    t0 = time.perf_counter()
    for a, b in ev:
        m.quantize(q, k, v)
        a.record(stream)
        m.attention()
        b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall / args.steps * 1e3
    attn_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    quant_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                for _ in range(args.steps)]
    for a, b in quant_ev:
        a.record(stream)
        m.quantize(q, k, v)
        b.record(stream)
    torch.cuda.synchronize()
    quant_ms = float(np.mean([a.elapsed_time(b) for a, b in quant_ev]))
    # the same with the 256 MB last-level cache flushed before every call (a 512 MB write), so
    # the quantizers read their inputs from HBM
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    cold = []
    for _ in range(min(args.steps, 20)):
        flush.fill_(1)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        m.quantize(q, k, v)
        b.record(stream)
        torch.cuda.synchronize()
        cold.append(a.elapsed_time(b))
    del flush
    quant_cold_ms = float(np.median(cold))

    flops = c.flops
    value = flops / (ms_per_step * 1e-3) / 1e12
    attn_tflops = flops / (attn_ms * 1e-3) / 1e12
    # algorithmic bytes of the quantize step per element of each tensor: FP8 mode, bf16 in + FP8
    # out (V transposed); FP4 mode, Q and K bf16 in + codes and scales (+ FP8 unless BMM1 takes
    # the FP4 form), V bf16 in + codes, scales and bf16 dequant, then the transposed FP8 pass
    n = c.B * c.H * c.N * c.d
    fp4_out = 0.5 + 1.0 / 32
    if c.mode == "fp8":
        quant_bytes = 3 * n * 3
    else:
        qk = 2 + fp4_out + (0 if args.native_fp4 else 1)
        quant_bytes = n * (2 * qk + (2 + fp4_out + 2) + 3)
    out = {
        "metric": "quantized SDPA TFLOP/s @ N=8704,H=24,d=128 + % of MI355X FP8 MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3",
        "data": "synthetic",
        "config": {"workload": c.name, "B": c.B, "H": c.H, "N": c.N, "d": c.d, "mode": c.mode,
                   "bmm1": ("mxfp4 codes on the scaled fp4 mfma" if args.native_fp4 else
                            "e4m3 values on the bf16 mfma"), "p_reading": args.p_reading,
                   "step": ("FP4 quantize Q,K,V (V then FP8) + attention with MXFP4 BMM1"
                            if args.native_fp4 else
                            "quantize Q,K,V to FP8 + fused attention (static scales)")},
        "roofline": {"bound": "mfma", "achieved": round(attn_tflops, 2),
                     "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(attn_tflops / FP8_PEAK_TFLOPS, 4),
                     "traffic": traffic_bytes() if (args.config == 3 and not args.native_fp4
                                                    and args.p_reading == "r3"
                                                    and args.heads is None) else None},
        "pct_fp8_peak_step": round(100 * value / FP8_PEAK_TFLOPS, 2),
        "attention_ms": round(attn_ms, 4),
        "quantize_ms": round(quant_ms, 4),
        "quantize_gbs": round(quant_bytes / (quant_ms * 1e-3) / 1e9, 1),
        "quantize_ms_cache_flushed": round(quant_cold_ms, 4),
        "quantize_gbs_cache_flushed": round(quant_bytes / (quant_cold_ms * 1e-3) / 1e9, 1),
    }
    if not args.no_cpu_baseline:
        out["host_cpu"] = host_cpu()
        out["cpu_baseline"] = cpu_baseline(args.config, args.cpu_seconds)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
