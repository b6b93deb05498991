"""bench.py's command-line contract: one JSON line with the documented keys, and a refusal of
more than one GPU before anything touches a device."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args, timeout=240):
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                       capture_output=True, text=True, timeout=timeout)
    lines = [l for l in p.stdout.splitlines() if l.strip()]
    return p.returncode, lines, p.stderr


def test_bench_refuses_several_gpus():
    rc, lines, _ = _run("--gpus", "2", timeout=60)
    assert rc == 2
    assert len(lines) == 1 and "one GPU" in json.loads(lines[0])["error"]


def _check_common(d, steps, warmup):
    assert d["n_gpus"] == 1 and d["steps"] == steps and d["warmup"] == warmup
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["unit"] == "TFLOP/s"
    assert d["higher_is_better"] is True and d["scaling"] == "weak" and d["vs_baseline"] is None
    assert d["data"] == "synthetic" and isinstance(d["dtype"], str)
    assert isinstance(d["config"]["workload"], str)
    r = d["roofline"]
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s" and r["peak"] > 0
    assert r["achieved"] > 0 and abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-3
    assert r["traffic"] is None or r["traffic"] > 0


@pytest.mark.gpu
def test_bench_attention_line():
    print("bench: attention line, small workload", flush=True)
    rc, lines, err = _run("--config", "1", "--steps", "3", "--warmup", "2", "--cpu-seconds", "1",
                          "--ramp-seconds", "0.05")
    assert rc == 0, err[-2000:]
    assert len(lines) == 1
    d = json.loads(lines[0])
    _check_common(d, 3, 2)
    assert d["config"]["N"] == 256 and d["roofline"]["traffic"] is None   # counters: bench shape only
    mc = d["roofline_mixed_ceiling"]
    assert mc["peak"] > d["roofline"]["peak"] / 2 and mc["frac"] > d["roofline"]["frac"]
    assert d["clock_ramp"]["steps"] >= 20
    for name in ("amax_bf16", "fp8_rows", "fp8_transposed", "fp4_block", "fp4_block_fp8"):
        kd = d["quantizer_kernels_cold"][name]
        assert kd["us"] > 0 and kd["gbs"] > 0
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1
    assert cb["unit"] == "TFLOP/s" and isinstance(cb["sample"], str)
    par = d["parity_sampled_rows"]
    assert par["rows"] > 0 and par["rel_l2_vs_oracle"] <= 1e-2 and par["max_abs_vs_oracle"] <= 5e-2
    assert 0 < par["rel_l2_vs_fp64_unquantized"] < 0.5


@pytest.mark.gpu
def test_bench_gemm_line():
    print("bench: GEMM line, output projection", flush=True)
    rc, lines, err = _run("--gemm", "fp8", "--gemm-shape", "out", "--steps", "3", "--warmup", "2",
                          "--no-cpu-baseline")
    assert rc == 0, err[-2000:]
    assert len(lines) == 1
    d = json.loads(lines[0])
    _check_common(d, 3, 2)
    assert "cpu_baseline" not in d
