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
BF16_PEAK_TFLOPS = 2500.0     # MI355X dense bf16 MFMA peak
HBM_PEAK_GBS = 8000.0
# BMM1 runs on the bf16 matrix instruction (gfx950's FP8 forms truncate the products), BMM2 on
# the FP8 one: equal FLOPs at 2.5 and 5.0 PFLOP/s bound the attention at their harmonic mean
MIXED_PEAK_TFLOPS = 2.0 / (1.0 / BF16_PEAK_TFLOPS + 1.0 / FP8_PEAK_TFLOPS)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=150)
    # the shader clock under this load takes ~0.1 s of continuous work to settle (and an idle
    # box starts low), so untimed steps run for this long before the warm-up steps
    ap.add_argument("--ramp-seconds", type=float, default=0.5)
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
    ap.add_argument("--svdquant-rank", type=int, default=0,
                    help="with --gemm mxfp4: SVD-Quant in FP4, a rank-r bf16 branch plus the "
                         "MXFP4 GEMM of the residual (weights with a planted low-rank part)")
    ap.add_argument("--gemm-out", choices=["f32", "bf16"], default="f32",
                    help="C in float32 (kq_gemm_*) or bf16 (kq_gemm_*_bf16)")
    ap.add_argument("--quantizers", action="store_true",
                    help="only the per-kernel quantizer timing (inputs read from HBM: copies in "
                         "rotation), one JSON line; the command profiled for the quantizer kernels")
    ap.add_argument("--pmc-workload", action="store_true",
                    help="no timing: a plain copy of COPY_BYTES (counter calibration), then "
                         "--pmc-steps steps; run under rocprofv3 --pmc")
    ap.add_argument("--pmc-steps", type=int, default=3)
    ap.add_argument("--trace-summary", nargs="+", metavar=("CSV", "SKIP"), default=None,
                    help="no GPU: a rocprofv3 kernel_trace.csv (and optionally how many first "
                         "calls of each kernel to drop as warm-up); prints per-kernel "
                         "statistics and the kernel sources' digests")
    ap.add_argument("--pmc-summary", nargs="+", metavar=("KIND", "CSV"), default=None,
                    help="no GPU: KIND 'traffic', 'counters' or 'gemm', then rocprofv3 "
                         "counter_collection.csv files of --pmc-workload runs; prints the "
                         "summary kept under profiles/")
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


def _short_kernel_name(name: str) -> str:
    name = name.replace("(anonymous namespace)::", "").replace("void ", "")
    return name.split("(")[0].split("::")[-1]


def _read_counters(paths):
    """{kernel: {counter: [value per dispatch]}} and {kernel: [duration ns per dispatch]}."""
    import csv
    vals, durs = {}, {}
    for path in paths:
        seen = set()
        with open(path) as f:
            for r in csv.DictReader(f):
                k = _short_kernel_name(r["Kernel_Name"])
                vals.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(
                    float(r["Counter_Value"]))
                key = (k, r["Dispatch_Id"])
                if key not in seen:
                    seen.add(key)
                    durs.setdefault((path, k), []).append(
                        int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    return vals, durs


def source_sha(name: str) -> str:
    import hashlib
    with open(os.path.join(ROOT, "precision_quantized_attention_amd", "csrc", name), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


# algorithmic bytes per element of each quantizer kernel (inputs read once, outputs written
# once): bf16 in; FP8 out 1; FP4 codes 0.5 + E8M0 1/32; fused FP8 1; dequantized bf16 2
QUANT_BYTES = {"amax_bf16_kernel": 2.0, "fp8_rows_kernel": 3.0, "fp8_transposed_kernel": 3.0,
               "fp4_block_kernel<false, false, false>": 2.53125,
               "fp4_block_kernel<false, false, true>": 3.53125,
               "fp4_block_kernel<false, true, false>": 4.53125,
               "fp4_block_kernel<true, false, true>": 3.53125}


def trace_summary(path, skip=0, elements=0):
    """Per-kernel duration statistics of a rocprofv3 --kernel-trace CSV (microseconds), with the
    digests of the kernel sources; with skip > 0 also each kernel's statistics past its first
    `skip` calls; with elements > 0 the GB/s of each quantizer kernel on a tensor of that many
    elements (algorithmic bytes / median duration)."""
    import csv
    import statistics
    d = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            name = r["Kernel_Name"].replace("(anonymous namespace)::", "")
            name = name.split("(")[0] if not name.startswith("void at::") else name[:60]
            d.setdefault(name, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    tot = sum(sum(v) for v in d.values())
    out = [f"# kernel sources sha256[:16]: attn_fp8.hip {source_sha('attn_fp8.hip')}, "
           f"gemm.hip {source_sha('gemm.hip')}, quant.hip {source_sha('quant.hip')}",
           f"{'kernel':62s} {'calls':>6s} {'avg_us':>9s} {'median_us':>9s} {'min_us':>8s} "
           f"{'max_us':>8s} {'pct':>6s}"]
    for k, v in sorted(d.items(), key=lambda kv: -sum(kv[1])):
        out.append(f"{k[:62]:62s} {len(v):6d} {statistics.mean(v):9.2f} {statistics.median(v):9.2f} "
                   f"{min(v):8.2f} {max(v):8.2f} {100 * sum(v) / tot:6.2f}")
    if skip:
        for k, v in sorted(d.items(), key=lambda kv: -sum(kv[1])):
            if len(v) > skip:
                w = v[skip:]
                out.append(f"# {k[:62]}: past its first {skip} calls, {len(w)} calls, mean "
                           f"{statistics.mean(w):.2f} us, median {statistics.median(w):.2f} us")
    if elements:
        out.append(f"# GB/s = {elements} elements x bytes per element / median duration "
                   f"(HBM peak {HBM_PEAK_GBS:.0f})")
        for k, v in d.items():
            base = k.replace("void ", "").split("::")[-1]
            b = next((b for pat, b in QUANT_BYTES.items()
                      if base == pat or ("<" not in pat and base.split("<")[0] == pat)), None)
            if b is not None:
                med = statistics.median(v)
                gbs = elements * b / (med * 1e-6) / 1e9
                out.append(f"{k[:62]:62s} {b:7.4f} B/elem {gbs:8.1f} GB/s "
                           f"{100 * gbs / HBM_PEAK_GBS:5.1f}%")
    return "\n".join(out)


def pmc_summary(kind, paths):
    """Text summary of --pmc-workload counter runs (one rocprofv3 pass per CSV).

    traffic: FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of every kernel, scaled by what they
    read for the plain 1 GiB copy that opens the run (the largest __amd_rocclr_copyBuffer
    dispatch), as bytes per launch (median over dispatches).
    counters: the attention kernel's SQ/GRBM counters (medians over the dispatches past the
    first five, whose clock is still rising) and the figures derived from them.
    gemm: the same for the projection GEMM kernel (a `--gemm ... --pmc-workload` run)."""
    import statistics
    vals, durs = _read_counters(paths)
    med = lambda v: statistics.median(v[5:] if len(v) > 5 else v)
    out = [f"kernel_sha: {kernel_sha()}"]
    if kind == "traffic":
        copy = vals["__amd_rocclr_copyBuffer"]
        fscale = COPY_BYTES / (max(copy["FETCH_SIZE"]) * 1024) if "FETCH_SIZE" in copy else None
        wscale = COPY_BYTES / (max(copy["WRITE_SIZE"]) * 1024) if "WRITE_SIZE" in copy else None
        out += [f"copy_fetch_scale: {fscale:.4f}", f"copy_write_scale: {wscale:.4f}"]
        for k in sorted(vals):
            if not k.startswith(("attn", "amax", "fp8", "fp4")):
                continue
            name = "attn" if k.startswith("attn_fp8_kernel") else k.split("<")[0]
            for ctr, sc, tag in (("FETCH_SIZE", fscale, "fetch"), ("WRITE_SIZE", wscale, "write")):
                if ctr in vals[k]:
                    out.append(f"{name}_{tag}_bytes_per_launch: "
                               f"{round(med(vals[k][ctr]) * 1024 * sc)}")
        return "\n".join(out)
    # counters of the attention kernel ("counters") or of the projection GEMM ("gemm")
    gemm = kind == "gemm"
    k = next(n for n in vals if n.startswith("gemm_kernel" if gemm else "attn_fp8_kernel"))
    if gemm:
        out[0] = f"kernel_sha: {source_sha('gemm.hip')}  (gemm.hip)"
    c = {ctr: med(v) for ctr, v in vals[k].items()}
    dur_ns = statistics.median(d for (p, n), ds in durs.items() if n == k
                               for d in (ds[5:] if len(ds) > 5 else ds))
    xcds, cus, simds = 8, 256, 1024
    cyc = c["GRBM_GUI_ACTIVE"] / xcds            # GRBM_GUI_ACTIVE is summed over the XCDs
    out.append(f"kernel: {k}")
    out.append(f"duration_us: {dur_ns / 1e3:.1f}")
    for ctr in sorted(c):
        out.append(f"{ctr}: {c[ctr]:.0f}")
    out.append(f"gpu_clock_ghz: {cyc / dur_ns:.3f}  (GRBM_GUI_ACTIVE / {xcds} XCDs / duration)")
    if "SQ_VALU_MFMA_BUSY_CYCLES" in c:
        out.append(f"mfma_busy_pct: {100 * c['SQ_VALU_MFMA_BUSY_CYCLES'] / (cyc * simds):.1f}"
                   f"  (SQ_VALU_MFMA_BUSY_CYCLES / (cycles x {simds} SIMDs))")
    if "SQ_ACTIVE_INST_VALU" in c:
        out.append(f"valu_busy_pct: {100 * c['SQ_ACTIVE_INST_VALU'] / (cus * cyc):.1f}"
                   f"  (SQ_ACTIVE_INST_VALU / {cus} CUs / cycles)")
    if "SQ_WAIT_INST_ANY" in c and "SQ_WAVE_CYCLES" in c:
        out.append(f"wave_wait_pct: {100 * c['SQ_WAIT_INST_ANY'] / c['SQ_WAVE_CYCLES']:.1f}"
                   f"  (SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES: waves waiting on a dependency)")
    if gemm:
        if "SQ_LDS_BANK_CONFLICT" in c and "SQ_LDS_IDX_ACTIVE" in c:
            out.append(f"lds_bank_conflict_pct: "
                       f"{100 * c['SQ_LDS_BANK_CONFLICT'] / c['SQ_LDS_IDX_ACTIVE']:.1f}"
                       f"  (SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE)")
        return "\n".join(out)
    if "SQ_VALU_MFMA_COEXEC_CYCLES" in c and "SQ_VALU_MFMA_BUSY_CYCLES" in c:
        out.append(f"valu_coexec_pct_of_mfma_busy: "
                   f"{100 * c['SQ_VALU_MFMA_COEXEC_CYCLES'] / c['SQ_VALU_MFMA_BUSY_CYCLES']:.1f}")
    # per wave-tile (32 query rows x 64 keys) of the FLUX.1 Kontext workload the runs use
    import workloads as W
    w = W.config(3)
    tiles = w.B * w.H * -(-w.N // 32) * -(-w.N // 64)
    out.append(f"wave_tiles: {tiles}")
    for ctr, tag in (("SQ_INSTS_VALU", "valu_insts"), ("SQ_INSTS_MFMA", "mfma_insts"),
                     ("SQ_INSTS_VALU_TRANS_F32", "trans_insts"), ("SQ_INSTS_VALU_CVT", "cvt_insts"),
                     ("SQ_INSTS_LDS", "lds_insts"), ("SQ_INSTS_SALU", "salu_insts")):
        if ctr in c:
            out.append(f"{tag}_per_wave_tile: {c[ctr] / tiles:.1f}")
    if "SQ_ACTIVE_INST_VALU" in c:
        out.append(f"valu_active_cycles_per_wave_tile: {4 * c['SQ_ACTIVE_INST_VALU'] / tiles:.0f}"
                   f"  (SQ_ACTIVE_INST_VALU counts quad-cycles)")
    if "SQ_VALU_MFMA_BUSY_CYCLES" in c:
        out.append(f"mfma_busy_cycles_per_wave_tile: {c['SQ_VALU_MFMA_BUSY_CYCLES'] / tiles:.0f}")
    out.append(f"simd_cycles_per_wave_tile: {cyc * simds / tiles:.0f}")
    if "SQ_LDS_BANK_CONFLICT" in c and "SQ_LDS_IDX_ACTIVE" in c:
        out.append(f"lds_bank_conflict_pct: "
                   f"{100 * c['SQ_LDS_BANK_CONFLICT'] / c['SQ_LDS_IDX_ACTIVE']:.1f}"
                   f"  (SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE)")
    return "\n".join(out)


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


def blas_threads() -> int:
    """Threads of the BLAS library numpy's matrix products run on (the oracle's products)."""
    try:
        from threadpoolctl import threadpool_info
        n = [i["num_threads"] for i in threadpool_info() if i.get("user_api") == "blas"]
        if n:
            return int(max(n))
    except Exception:
        pass
    return 1


def host_cores() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        return os.cpu_count() or 1


def cpu_baseline(cfg, target_s, gpu_o=None, heads=None):
    """Time the CPU oracle (as it stands) on a bounded sample of the workload: the full
    per-tensor quantization of Q, K, V, then R3 attention for query rows of successive heads
    until about `target_s` seconds have been spent.

    With gpu_o (the GPU output [B, H, N, d] of one forward on the same inputs) also returns the
    GPU's error on the sampled rows: against the oracle (the parity gate's metrics) and against
    unquantized float64 attention of the bf16 inputs (reported, not gated; its rows are the
    first 256 of each sampled head, computed after the timing)."""
    import numpy as np
    import workloads as W
    from oracle import attention as A
    from oracle import pipeline as OP

    c = W.config(cfg)
    H = c.H if heads is None else heads
    pos = W.positions(c) if c.rope else None
    bits = W.qkv_bits(cfg)
    if heads is not None:
        bits = tuple(np.ascontiguousarray(b[:, :heads]) for b in bits)
    t0 = time.perf_counter()
    qz = OP.quantize_inputs(*bits, mode=c.mode, positions=pos)
    t_quant = time.perf_counter() - t0
    rows_done, t_attn = 0, 0.0
    done = []                        # (b, h, rows, O) of the timed sample
    sm = np.float32(1 / math.sqrt(c.d))
    for b in range(c.B):
        for h in range(H):
            if rows_done and t_attn + t_quant >= target_s:
                break
            sl = (slice(b, b + 1), slice(h, h + 1))
            for r0 in range(0, c.N, 1024):
                if rows_done and t_attn + t_quant >= target_s:
                    break
                rows = np.arange(r0, min(c.N, r0 + 1024))
                t0 = time.perf_counter()
                O, _, _ = A.attention_r3(qz.codes["q"][sl], qz.codes["k"][sl], qz.codes["v"][sl],
                                         qz.scale["q"][0], qz.scale["k"][0], qz.scale["v"][0], sm,
                                         rows=rows)
                t_attn += time.perf_counter() - t0
                rows_done += len(rows)
                done.append((b, h, rows, O[0, 0]))
    # attention FLOPs of the processed rows (4*N*d each) per second; the quantization of the
    # whole tensors is charged in proportion to the rows processed
    total_rows = c.B * H * c.N
    flops = 4.0 * rows_done * c.N * c.d
    t = t_attn + t_quant * rows_done / total_rows
    heads_done = len({(b, h) for b, h, _, _ in done})
    base = {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": blas_threads(),
            "kind": "oracle",
            "sample": f"{c.name}: quantization of the full Q, K, V ({t_quant:.1f} s) and R3 "
                      f"attention for {rows_done} query rows in {heads_done} heads "
                      f"({t_attn:.1f} s); quantization charged pro rata; numpy float64 products "
                      f"on {blas_threads()} BLAS threads of {host_cores()} host cores"}
    if gpu_o is None:
        return base, None
    num = den = 0.0
    mab = 0.0
    for b, h, rows, O in done:
        g = gpu_o[b, h, rows].astype(np.float64)
        num += float(np.sum((g - O) ** 2))
        den += float(np.sum(O.astype(np.float64) ** 2))
        mab = max(mab, float(np.max(np.abs(g - O))))
    # float64 attention of the unquantized (bf16) inputs, first 256 rows of each sampled head
    # (after RoPE where the workload has it: the rotation is part of the model, not of the
    # quantization)
    fnum = fden = 0.0
    n64 = 0
    for b, h in sorted({(b, h) for b, h, _, _ in done}):
        rows = np.arange(min(256, c.N))
        xs = [qz.x[n][b:b + 1, h:h + 1] for n in "qkv"]
        if c.mode == "fp4":        # qz.x holds the FP4-dequantized tensors: start from bf16
            from oracle import formats as Fm
            from oracle import rope as R
            xs = [Fm.bf16_bits_to_f32(x[b:b + 1, h:h + 1]) for x in bits]
            if pos is not None:
                tab = R.table(pos)
                xs[0], xs[1] = R.apply(xs[0], tab), R.apply(xs[1], tab)
        ref = A.attention_fp64(*xs, float(sm), rows=rows)[0, 0]
        g = gpu_o[b, h, rows].astype(np.float64)
        fnum += float(np.sum((g - ref) ** 2))
        fden += float(np.sum(ref ** 2))
        n64 += len(rows)
    parity = {"rows": rows_done, "rel_l2_vs_oracle": math.sqrt(num / den),
              "max_abs_vs_oracle": mab, "rel_l2_vs_fp64_unquantized": math.sqrt(fnum / fden),
              "fp64_rows": n64}
    return base, parity


def gemm_main(args):
    """One JSON line for a projection GEMM: a step is one kq_gemm_* launch on codes prepared
    (quantized by the library's own kernels) before the timed region.  With --svdquant-rank r
    (MXFP4 only) the weights carry a planted low-rank part, the library's offline step splits
    them into bf16 rank-r factors and a residual (untimed), and a step is the branch's
    down-projection plus the fused GEMM."""
    import numpy as np
    import torch
    import workloads as W
    import precision_quantized_attention_amd as kq
    from precision_quantized_attention_amd.pipeline import bf16_from_bits

    shape = W.GEMM_SHAPES[0 if args.gemm_shape == "qkv" else 1]
    M, N, K = shape.M, shape.N, shape.K
    rank = args.svdquant_rank
    if rank and args.gemm != "mxfp4":
        print(json.dumps({"error": "--svdquant-rank needs --gemm mxfp4"}))
        sys.exit(2)
    torch.cuda.set_device(0)
    seed = 100 + N
    a_bits, w_bits = W.gemm_bits(M, N, K, seed)
    t_prep = 0.0
    if rank:
        w_bits = W.lowrank_weight_bits(N, K, seed + 7)
        t0 = time.perf_counter()
        lu_bits, ld_bits, r_bits = kq.kq_svdquant_factorize(w_bits, rank)   # offline, host
        t_prep = time.perf_counter() - t0
        l_up, l_down = bf16_from_bits(lu_bits), bf16_from_bits(ld_bits)
    a, w = bf16_from_bits(a_bits), bf16_from_bits(r_bits if rank else w_bits)
    bf16_out = args.gemm_out == "bf16"
    c = torch.empty((M, N), dtype=torch.bfloat16 if bf16_out else torch.float32, device="cuda")
    flops = shape.flops + (2 * M * rank * (K + N) if rank else 0)
    down = None
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
        if rank:
            # per forward: one pass over the activations (their MXFP4 codes and the branch's
            # T), then the fused GEMM
            t = torch.empty((M, rank), dtype=torch.bfloat16, device="cuda")
            gemm = kq.kq_gemm_mxfp4_svdquant_bf16 if bf16_out else kq.kq_gemm_mxfp4_svdquant
            down = lambda: kq.kq_svdquant_activations(a, l_down, ac, asc, t)
            launch = lambda: gemm(ac, asc, wc, wsc, t, l_up, c)
        else:
            gemm = kq.kq_gemm_mxfp4_bf16 if bf16_out else kq.kq_gemm_mxfp4
            launch = lambda: gemm(ac, asc, wc, wsc, c)
        peak = FP4_PEAK_TFLOPS
    stream = torch.cuda.current_stream()

    def step():
        if down is not None:
            down()
        launch()

    if args.pmc_workload:
        src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        for _ in range(args.pmc_steps):
            step()
        torch.cuda.synchronize()
        print(json.dumps({"pmc_workload": shape.name, "copy_bytes": COPY_BYTES,
                          "steps": args.pmc_steps}))
        return
    ramp(step, args.ramp_seconds)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # timed steps; HIP events on the launch stream bracket the GEMM launch (and the branch's
    # down-projection) inside the timed region
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for e0, e1, e2 in ev:
        e0.record(stream)
        if down is not None:
            down()
        e1.record(stream)
        launch()
        e2.record(stream)
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) / args.steps * 1e3
    kern_ms = float(np.mean([e1.elapsed_time(e2) for e0, e1, e2 in ev]))
    down_ms = float(np.mean([e0.elapsed_time(e1) for e0, e1, e2 in ev])) if rank else 0.0
    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = (flops - (2 * M * rank * K if rank else 0)) / (kern_ms * 1e-3) / 1e12
    if rank:
        fmt_name = f"SVD-Quant FP4: MXFP4 residual + rank-{rank} bf16 branch"
    else:
        fmt_name = "FP8 E4M3 per-tensor (W8A8)" if args.gemm == "fp8" else "MXFP4 (E2M1, E8M0 per 32)"
    out = {
        "metric": f"quantized projection GEMM TFLOP/s ({fmt_name})",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8_e4m3" if args.gemm == "fp8" else "mxfp4_e2m1", "data": "synthetic",
        "config": {"workload": shape.name + (f"_svdquant_r{rank}" if rank else ""), "M": M,
                   "N": N, "K": K, "rank": rank,
                   "step": ("activation pass (MXFP4 codes of A + branch down-projection) + fused "
                            "GEMM (MXFP4 residual + branch), " if rank
                            else "one GEMM launch on prepared codes, ")
                           + ("bf16 C" if bf16_out else "float32 C")},
        # the GEMM launch alone: its MXFP4 FLOPs plus the branch's up-projection, at the FP4 peak
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": None},
        "gemm_ms": round(kern_ms, 4),
    }
    if args.gemm == "fp8" and not rank:
        # the vendor library on the same codes and scales (hipBLASLt through torch._scaled_mm),
        # timed the same way right after, alternating with this kernel; and whether its result
        # equals this kernel's bit for bit
        f8 = torch.float8_e4m3fn
        a_f8, w_f8 = a8.view(f8), w8.view(f8)
        s_a = torch.tensor(sa, dtype=torch.float32, device="cuda")
        s_w = torch.tensor(sw, dtype=torch.float32, device="cuda")
        odt = torch.bfloat16 if bf16_out else torch.float32
        vendor = lambda: torch._scaled_mm(a_f8, w_f8.t(), scale_a=s_a, scale_b=s_w, out_dtype=odt)
        try:
            ref = vendor()
            for _ in range(args.warmup):
                vendor()
            ours_us, theirs_us = [], []
            for _ in range(3):
                for fn, acc in ((launch, ours_us), (vendor, theirs_us)):
                    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                           for _ in range(args.steps)]
                    for e0, e1 in evs:
                        e0.record(stream)
                        fn()
                        e1.record(stream)
                    torch.cuda.synchronize()
                    acc.extend(e0.elapsed_time(e1) * 1e3 for e0, e1 in evs)
            launch()
            torch.cuda.synchronize()
            out["vendor_gemm"] = {
                "library": "hipBLASLt via torch._scaled_mm", "us": round(float(np.median(theirs_us)), 2),
                "this_kernel_us": round(float(np.median(ours_us)), 2),
                "ratio": round(float(np.median(ours_us) / np.median(theirs_us)), 4),
                "bit_identical": bool(torch.equal(ref, c)),
            }
        except (RuntimeError, TypeError) as e:          # no FP8 GEMM in this torch build
            out["vendor_gemm"] = {"error": str(e)[:200]}
    if rank:
        # the activation pass: A read once, its codes and scales and T written
        out["svdquant_activations_ms"] = round(down_ms, 4)
        out["svdquant_activations_gbs"] = round(
            M * (K * (2 + 0.5 + 1.0 / 32) + 2 * rank) / (down_ms * 1e-3) / 1e9, 1)
        out["svdquant_factorize_host_s"] = round(t_prep, 2)
    if not args.no_cpu_baseline:
        out["host_cpu"] = host_cpu()
        out["cpu_baseline"] = gemm_cpu_baseline(args.gemm, shape, a_bits, w_bits,
                                                args.cpu_seconds, rank=rank)
    print(json.dumps(out))


def gemm_cpu_baseline(fmt, shape, a_bits, w_bits, target_s, rank=0):
    """The oracle GEMM (exact float64) on successive 64-row blocks of the activations against
    all weights, quantized by the oracle, until about `target_s` seconds.  SVD-Quant: the
    oracle's offline weight step (float64 SVD, not charged: it is not part of the forward),
    then its forward on successive 64-row blocks."""
    import numpy as np
    import workloads as W
    from oracle import gemm as OG
    from oracle import quant as Qz

    if rank:
        from oracle import svdquant as OS
        t0 = time.perf_counter()
        prep = OS.quantize_weights(W.bits_to_f32(w_bits), rank)
        t_off = time.perf_counter() - t0
        rows, t = 0, 0.0
        while (t < target_s or rows == 0) and rows < shape.M:
            af = W.bits_to_f32(a_bits[rows:rows + 64])
            t0 = time.perf_counter()
            OS.forward(af, prep[0], prep[1], prep[3], prep[4])
            t += time.perf_counter() - t0
            rows += len(af)
        flops = 2.0 * rows * (shape.N * shape.K + rank * (shape.K + shape.N))
        return {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": blas_threads(),
                "kind": "oracle",
                "sample": f"{shape.name} SVD-Quant r={rank}: oracle forward (FP4 quantization "
                          f"of the rows, exact GEMM, bf16 branch) of {rows} activation rows "
                          f"({t:.1f} s); the offline weight step ({t_off:.1f} s) not charged; "
                          f"numpy float64 products on {blas_threads()} BLAS threads of "
                          f"{host_cores()} host cores"}
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
            "cores": blas_threads(), "kind": "oracle",
            "sample": f"{shape.name}: oracle quantization of the weights ({t_w:.1f} s, charged "
                      f"pro rata) and the exact GEMM of {rows} activation rows ({t:.1f} s); "
                      f"numpy float64 products on {blas_threads()} BLAS threads of "
                      f"{host_cores()} host cores"}


def ramp(step, seconds):
    """Untimed steps for at least `seconds` of wall time (the GPU kept busy throughout), so the
    timed steps run at the clock this load settles to rather than at the ramp from idle."""
    import torch
    n, t0 = 0, time.perf_counter()
    while True:
        for _ in range(20):
            step()
        n += 20
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= seconds:
            return n, time.perf_counter() - t0


def cold_launch_us(fns, stream, rounds=3, repeats=5):
    """Mean duration in microseconds of one launch that reads its inputs from HBM.  Each of
    `fns` works on its own copy of the inputs and outputs, the copies together well above the
    256 MB last-level cache, and they are launched in rotation, `rounds` times through the set
    back to back between one pair of HIP events on `stream`, so a copy has left the cache before
    it comes round again and the events' own overhead is spread over many launches.  Median of
    `repeats` such runs after one untimed pass."""
    import numpy as np
    import torch

    for f in fns:
        f()
    ts = []
    for _ in range(repeats):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(rounds):
            for f in fns:
                f()
        b.record(stream)
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b) * 1e3 / (rounds * len(fns)))
    return float(np.median(ts))


COLD_SETS = 8   # copies of a 53.5 MB tensor in rotation: 428 MB, above the 256 MB cache


def quantizer_rates(c, q, k, v, m, stream, rounds=3):
    """Each quantizer and calibration kernel of the workload with its input read from HBM
    (`cold_launch_us`: COLD_SETS copies of input and output in rotation): microseconds and GB/s
    of algorithmic bytes (inputs read once, outputs written once).  The FP4 encoder is also timed
    on the FP8 workloads' Q (codes + scales, and with the fused FP8 output), as the encoder of
    the FP4 variant on the same tensor size."""
    import torch
    import precision_quantized_attention_amd as kq

    n = q.numel()
    out = {}
    qs = [q.clone() for _ in range(COLD_SETS)]

    def timed(name, fns, bytes_per_elem):
        us = cold_launch_us(fns, stream, rounds=rounds)
        out[name] = {"us": round(us, 2), "gbs": round(n * bytes_per_elem / (us * 1e-6) / 1e9, 1),
                     "bytes_per_elem": round(bytes_per_elem, 4)}

    def outs(shape, dtype):
        return [torch.empty(shape, dtype=dtype, device="cuda") for _ in range(COLD_SETS)]

    am = torch.zeros(1, dtype=torch.float32, device="cuda")
    timed("amax_bf16", [lambda x=x: kq.kq_amax_calibrate(x, am) for x in qs], 2.0)
    inv_q = m.scales["q"][1]
    q8 = outs(q.shape, torch.uint8)
    timed("fp8_rows", [lambda x=x, y=y: kq.kq_quantize_fp8_tensor(x, inv_q, y)
                       for x, y in zip(qs, q8)], 3.0)
    vs = [v.clone() for _ in range(COLD_SETS)]
    vt = outs(m.buf.v8t.shape, m.buf.v8t.dtype)
    timed("fp8_transposed", [lambda x=x, y=y: kq.kq_quantize_fp8_tensor(
        x, m.scales["v"][1], y, layout=kq.KQ_LAYOUT_TRANSPOSED) for x, y in zip(vs, vt)], 3.0)
    del vs, vt
    d = q.shape[-1]
    codes = outs(q.shape[:-1] + (d // 2,), torch.uint8)
    scales = outs(q.shape[:-1] + (d // 32,), torch.uint8)
    enc = 2 + 0.5 + 1.0 / 32
    sets = list(zip(qs, codes, scales, q8))
    timed("fp4_block", [lambda x=x, cd=cd, sc=sc: kq.kq_quantize_fp4_block(x, cd, sc)
                        for x, cd, sc, _ in sets], enc)
    timed("fp4_block_fp8", [lambda x=x, cd=cd, sc=sc, y=y: kq.kq_quantize_fp4_block(
        x, cd, sc, fp8=y, inv_scale8=inv_q) for x, cd, sc, y in sets], enc + 1)
    if m.rope is not None:
        timed("fp4_block_rope_fp8", [lambda x=x, cd=cd, sc=sc, y=y: kq.kq_quantize_fp4_block(
            x, cd, sc, fp8=y, inv_scale8=inv_q, rope=m.rope) for x, cd, sc, y in sets], enc + 1)
    del q8
    dq = outs(q.shape, q.dtype)
    timed("fp4_block_dq", [lambda x=x, cd=cd, sc=sc, y=y: kq.kq_quantize_fp4_block(
        x, cd, sc, dq=y) for (x, cd, sc, _), y in zip(sets, dq)], enc + 2)
    return out


def main():
    args = parse()
    if args.pmc_summary:
        print(pmc_summary(args.pmc_summary[0], args.pmc_summary[1:]))
        return
    if args.trace_summary:
        skip = int(args.trace_summary[1]) if len(args.trace_summary) > 1 else 0
        elements = int(args.trace_summary[2]) if len(args.trace_summary) > 2 else 0
        print(trace_summary(args.trace_summary[0], skip, elements))
        return
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
        for _ in range(args.pmc_steps):
            m.forward(q, k, v)
        torch.cuda.synchronize()
        print(json.dumps({"pmc_workload": c.name, "copy_bytes": COPY_BYTES,
                          "steps": args.pmc_steps}))
        return

    if args.quantizers:
        rounds = max(1, args.steps // COLD_SETS)
        rates = quantizer_rates(c, q, k, v, m, stream, rounds=rounds)
        print(json.dumps({"quantizer_kernels_cold": rates, "workload": c.name,
                          "launches_per_kernel": COLD_SETS * (1 + 5 * rounds),
                          "hbm_peak_gbs": HBM_PEAK_GBS}))
        return

    ramp_steps, ramp_s = ramp(lambda: m.forward(q, k, v), args.ramp_seconds)
    for _ in range(args.warmup):
        m.forward(q, k, v)
    torch.cuda.synchronize()

    # timed steps (forward = the per-forward quantization, then attention; in FP8 mode K and V
    # through the quantizers and Q inside the attention kernel); HIP events on the attention's
    # stream bracket its launch inside each timed step
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    t0 = time.perf_counter()
    for a, b in ev:
        m.prepare(q, k, v)
        a.record(stream)
        m.attention()
        b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall / args.steps * 1e3
    attn_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    gpu_o = m.buf.o.cpu().numpy()            # output of the last timed step, for the parity keys
    quant_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                for _ in range(args.steps)]
    for a, b in quant_ev:
        a.record(stream)
        m.prepare(q, k, v)
        b.record(stream)
    torch.cuda.synchronize()
    quant_ms = float(np.mean([a.elapsed_time(b) for a, b in quant_ev]))
    # the same with Q, K and V read from HBM: COLD_SETS copies of them in rotation
    cold_sets = [(q.clone(), k.clone(), v.clone()) for _ in range(COLD_SETS)]
    quant_cold_ms = cold_launch_us([lambda t=t: m.prepare(*t) for t in cold_sets], stream) * 1e-3
    del cold_sets
    kernels = quantizer_rates(c, q, k, v, m, stream)

    flops = c.flops
    value = flops / (ms_per_step * 1e-3) / 1e12
    attn_tflops = flops / (attn_ms * 1e-3) / 1e12
    # algorithmic bytes of the quantize step per element of each tensor: FP8 mode, bf16 in + FP8
    # out (V transposed), for K and V (Q too when it is not quantized in the attention kernel);
    # FP4 mode, Q and K bf16 in + codes and scales (+ FP8 unless BMM1 takes the FP4 form), V bf16
    # in + codes, scales and bf16 dequant, then the transposed FP8 pass
    n = c.B * c.H * c.N * c.d
    fp4_out = 0.5 + 1.0 / 32
    if c.mode == "fp8":
        quant_bytes = (2 if m.fuse_q else 3) * n * 3
    else:
        qk = 2 + fp4_out + (0 if args.native_fp4 else 1)
        quant_bytes = n * (2 * qk + (2 + fp4_out + 2) + 3)
    bmm1 = "mxfp4" if args.native_fp4 else "bf16"
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
                            "quantize K,V to FP8 + fused attention quantizing bf16 Q to FP8 "
                            "in-kernel (static scales)" if m.fuse_q else
                            "quantize Q,K,V to FP8 + fused attention (static scales)")},
        "roofline": {"bound": "mfma", "achieved": round(attn_tflops, 2),
                     "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(attn_tflops / FP8_PEAK_TFLOPS, 4),
                     "traffic": traffic_bytes() if (args.config == 3 and not args.native_fp4
                                                    and args.p_reading == "r3"
                                                    and args.heads is None) else None},
        # the same achieved rate against the peak of the instructions the kernel can use: BMM1
        # on bf16 (FP8 truncates its products), BMM2 on FP8
        "roofline_mixed_ceiling": ({"peak": round(MIXED_PEAK_TFLOPS, 1), "unit": "TFLOP/s",
                                    "frac": round(attn_tflops / MIXED_PEAK_TFLOPS, 4),
                                    "bmm1": "bf16 2.5 PFLOP/s", "bmm2": "fp8 5.0 PFLOP/s"}
                                   if bmm1 == "bf16" else None),
        "pct_fp8_peak_step": round(100 * value / FP8_PEAK_TFLOPS, 2),
        "attention_ms": round(attn_ms, 4),
        "clock_ramp": {"steps": ramp_steps, "seconds": round(ramp_s, 3)},
        "quantize_ms": round(quant_ms, 4),
        "quantize_gbs": round(quant_bytes / (quant_ms * 1e-3) / 1e9, 1),
        "quantize_ms_cold": round(quant_cold_ms, 4),
        "quantize_gbs_cold": round(quant_bytes / (quant_cold_ms * 1e-3) / 1e9, 1),
        "quantizer_kernels_cold": kernels,
    }
    if not args.no_cpu_baseline:
        out["host_cpu"] = host_cpu()
        base, parity = cpu_baseline(args.config, args.cpu_seconds, gpu_o=gpu_o, heads=args.heads)
        out["cpu_baseline"] = base
        if parity is not None and args.p_reading == "r3" and not args.native_fp4:
            out["parity_sampled_rows"] = {k_: (round(v_, 8) if isinstance(v_, float) else v_)
                                          for k_, v_ in parity.items()}
    print(json.dumps(out))


if __name__ == "__main__":
    main()
