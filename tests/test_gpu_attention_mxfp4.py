"""GPU parity of the attention with a native MXFP4 BMM1 (kq_attn_mxfp4_fwd) against the oracle
(attention_r3_mxfp4): Q and K stay E2M1 + E8M0 (the FP4 quantizer's output, RoPE first where the
workload has it), V goes FP4 -> per-tensor FP8 as in the FP4 workloads.

The FP4 codes and scales and V's FP8 codes are compared bit-exactly, the output within the
attention gate (rel-L2 1e-2, max-abs 5e-2).  At full size the oracle evaluates sampled query
rows of three heads.
"""
import math

import numpy as np
import pytest
import torch

import precision_quantized_attention_amd as kq
import workloads as W
from kq_testutil import MAX_ABS_TOL, REL_L2_TOL, max_abs, rel_l2, sample_rows, to_dev
from oracle import attention as A
from oracle import pipeline as OP
from precision_quantized_attention_amd.pipeline import QuantizedSDPA

pytestmark = pytest.mark.gpu


def _run(bits, positions=None, stats=False):
    B, H, N, d = bits[0].shape
    x = [to_dev(b) for b in bits]
    m = QuantizedSDPA(B, H, N, d, mode="fp4", positions=positions, want_stats=stats,
                      native_fp4=True)
    m.calibrate(*x)
    o = m.forward(*x)
    torch.cuda.synchronize()
    return m, o


def _check_inputs(m, qz):
    for n in "qk":
        codes, scales = m.buf.fp4[n]
        assert np.array_equal(codes.cpu().numpy(), qz.fp4[n][0]), n
        assert np.array_equal(scales.cpu().numpy(), qz.fp4[n][1]), n
    assert m.scales["v"] == qz.scale["v"]
    B, H, N, d = qz.codes["v"].shape
    vt = m.buf.v8t.cpu().numpy()[:, :, :N].transpose(0, 2, 1).reshape(B, H, N, d)
    assert np.array_equal(vt, qz.codes["v"])


def _oracle(qz, heads, rows, sm):
    sel = lambda a: np.stack([a[b, h] for b, h in heads])[None]
    (qc, qs, _), (kc, ks, _) = qz.fp4["q"], qz.fp4["k"]
    return A.attention_r3_mxfp4(sel(qc), sel(qs), sel(kc), sel(ks), sel(qz.codes["v"]),
                                qz.scale["v"][0], sm, rows=rows)


def _compare(o_gpu, o_ref, label):
    e, a = rel_l2(o_gpu, o_ref), max_abs(o_gpu, o_ref)
    print(f"{label}: rel_l2 {e:.3e} max_abs {a:.3e} (|O| max {np.abs(o_ref).max():.3g})",
          flush=True)
    assert e <= REL_L2_TOL, (label, e)
    assert a <= MAX_ABS_TOL, (label, a)


@pytest.mark.parametrize("cfg", [4, 5])
def test_mxfp4_attention_config(cfg):
    c = W.config(cfg)
    print(f"mxfp4-bmm1 attention cfg{cfg} {c.name} B={c.B} H={c.H} N={c.N} rope={c.rope}",
          flush=True)
    bits = W.qkv_bits(cfg)
    pos = W.positions(c) if c.rope else None
    m, o = _run(bits, positions=pos, stats=True)
    qz = OP.quantize_inputs(*bits, mode="fp4", positions=pos)
    _check_inputs(m, qz)
    rows = sample_rows(c.N, 24, seed=40 + cfg)
    heads = [(0, 0), (c.B - 1, c.H - 1), (c.B // 2, 7 % c.H)]
    O, M, L = _oracle(qz, heads, rows, m.sm_scale)
    o_np = o.cpu().numpy()
    got = np.stack([o_np[b, h][rows] for b, h in heads])
    _compare(got, O[0], f"cfg{cfg} mxfp4-bmm1 vs oracle")
    stats = m.buf.stats.cpu().numpy()
    st = np.stack([stats[b, h][rows] for b, h in heads])
    assert np.all(np.abs(st[..., 0] - M[0]) <= 1)
    assert np.allclose(st[..., 1].astype(np.float64) * np.exp2(st[..., 0]),
                       L[0].astype(np.float64) * np.exp2(M[0]), rtol=1e-2)
    # reported: the FP8-BMM1 oracle on the same inputs (the pages' numerics)
    sub = {n: np.stack([qz.codes[n][b, h] for b, h in heads])[None] for n in "qkv"}
    O8, _, _ = A.attention_r3(sub["q"], sub["k"], sub["v"], qz.scale["q"][0], qz.scale["k"][0],
                              qz.scale["v"][0], m.sm_scale, rows=rows)
    print(f"cfg{cfg}: native MXFP4 BMM1 vs FP8 BMM1 (oracle): rel_l2 {rel_l2(O[0], O8[0]):.3e}",
          flush=True)


@pytest.mark.parametrize("N", [1, 5, 64, 65, 129, 257, 1000])
def test_mxfp4_attention_ragged_lengths(N):
    print(f"mxfp4-bmm1 ragged N={N}", flush=True)
    bits = [W.random_bits(1, 2, N, 128, seed=900 + 3 * N + t, outliers=(N > 100))
            for t in range(3)]
    m, o = _run(bits)
    qz = OP.quantize_inputs(*bits, mode="fp4")
    _check_inputs(m, qz)
    O, _, _ = _oracle(qz, [(0, 0), (0, 1)], np.arange(N), m.sm_scale)
    _compare(o.cpu().numpy()[0], O[0], f"N={N}")


def test_mxfp4_attention_every_code_and_scale_spread():
    """Q and K codes drawn over all 16 E2M1 codes (both zeros included) with E8M0 scales
    spread over 2^-6 .. 2^0 per block, fed straight to the entry point."""
    print("mxfp4-bmm1 all codes", flush=True)
    B, H, N = 1, 2, 300
    rng = np.random.default_rng(77)
    qc = rng.integers(0, 256, size=(B, H, N, 64), dtype=np.uint8)
    kc = rng.integers(0, 256, size=(B, H, N, 64), dtype=np.uint8)
    qs = rng.integers(121, 128, size=(B, H, N, 4), dtype=np.uint8)
    ks = rng.integers(121, 128, size=(B, H, N, 4), dtype=np.uint8)
    v8 = rng.integers(0, 0x7F, size=(B, H, N, 128), dtype=np.uint8) | \
        (rng.integers(0, 2, size=(B, H, N, 128), dtype=np.uint8) << 7)
    s_v, sm = 0.01, float(np.float32(1 / math.sqrt(128)))
    vt = np.zeros((B * H, 128, kq.kq_vt_ld(N)), np.uint8)
    vt[:, :, :N] = v8.reshape(B * H, N, 128).transpose(0, 2, 1)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    o = torch.empty((B, H, N, 128), dtype=torch.float32, device="cuda")
    kq.kq_attn_mxfp4_fwd(dev(qc), dev(qs), dev(kc), dev(ks), dev(vt), s_v, sm, o)
    O, _, _ = A.attention_r3_mxfp4(qc, qs, kc, ks, v8, np.float32(s_v), np.float32(sm))
    _compare(o.cpu().numpy(), O, "all codes")


@pytest.mark.parametrize("gain", [8.0, 16.0])
def test_mxfp4_attention_large_score_gaps(gain):
    """Score rows that jump by ~2^130 / ~2^260 after the first key tiles (the guarded rescale
    and the offset clamp in the MXFP4-BMM1 instance), single pass and key split."""
    print(f"mxfp4-bmm1 score gaps gain={gain}", flush=True)
    bits = W.score_gap_bits(2, 320, gain, seed=77 + int(gain))
    m, o = _run(bits)
    qz = OP.quantize_inputs(*bits, mode="fp4")
    _check_inputs(m, qz)
    O, M, _ = _oracle(qz, [(0, 0), (0, 1)], np.arange(320), m.sm_scale)
    assert M[0, :, ::2].min() > 100
    (qc, qs), (kc, ks) = m.buf.fp4["q"], m.buf.fp4["k"]
    o1 = torch.empty_like(o)
    kq.kq_attn_mxfp4_fwd(qc, qs, kc, ks, m.buf.v8t, m.scales["v"][0], m.sm_scale, o1, None)
    torch.cuda.synchronize()
    _compare(o1.cpu().numpy()[0], O[0], f"gap {gain} single pass")
    _compare(o.cpu().numpy()[0], O[0], f"gap {gain} key split")


@pytest.mark.parametrize("B,H,N", [(1, 3, 8704), (1, 2, 1000), (1, 2, 65)])
def test_mxfp4_attention_key_split_matches_single_pass(B, H, N):
    print(f"mxfp4-bmm1 split B={B} H={H} N={N}", flush=True)
    bits = [W.random_bits(B, H, N, 128, seed=1300 + t, outliers=True) for t in range(3)]
    m, o = _run(bits)
    nbytes = kq.kq_attn_workspace_size(B, H, N)
    (qc, qs), (kc, ks) = m.buf.fp4["q"], m.buf.fp4["k"]
    o1 = torch.empty_like(o)
    kq.kq_attn_mxfp4_fwd(qc, qs, kc, ks, m.buf.v8t, m.scales["v"][0], m.sm_scale, o1, None)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device="cuda")
    o2 = torch.empty_like(o)
    kq.kq_attn_mxfp4_fwd(qc, qs, kc, ks, m.buf.v8t, m.scales["v"][0], m.sm_scale, o2, ws)
    torch.cuda.synchronize()
    a, b = o1.cpu().numpy(), o2.cpu().numpy()
    print(f"split bytes {nbytes}: rel_l2 {rel_l2(b, a):.3e}", flush=True)
    assert rel_l2(b, a) <= 1e-5 and max_abs(b, a) <= 1e-3
    if N <= 1000:
        qz = OP.quantize_inputs(*bits, mode="fp4")
        O, _, _ = _oracle(qz, [(0, h) for h in range(H)], np.arange(N), m.sm_scale)
        _compare(b[0], O[0], f"split N={N}")


def test_mxfp4_pipeline_refuses_out_of_range_scores():
    # the MXFP4 BMM1 needs sm_scale log2(e) 128 max|dq(q)| max|dq(k)| < 2^20; inputs scaled by
    # 1000 exceed it (about 2.6e8), so calibration refuses them instead of launching
    print("mxfp4-bmm1 range check", flush=True)
    g = torch.Generator(device="cpu").manual_seed(1400)
    x = [(torch.randn(1, 2, 256, 128, generator=g) * 1000).to(torch.bfloat16).cuda()
         for _ in range(3)]
    m = QuantizedSDPA(1, 2, 256, 128, mode="fp4", native_fp4=True)
    with pytest.raises(kq.KQError, match="2\\^20"):
        m.calibrate(*x)
    m8 = QuantizedSDPA(1, 2, 256, 128, mode="fp4")
    m8.calibrate(*x)                 # the FP8 BMM1 takes any finite scales


def test_mxfp4_attention_past_the_precondition_stays_finite():
    """The entry point itself, fed scales past its |t| < 2^20 precondition (E8M0 bytes up to
    2^12, |t| up to ~2^33, still finite in float32): 448 p may leave the E4M3 range there, and
    the codes saturate at 448, so every output is finite (the values themselves are not
    compared: the fused exp2 argument no longer follows the definition)."""
    print("mxfp4-bmm1 past the precondition", flush=True)
    B, H, N = 1, 2, 320
    rng = np.random.default_rng(91)
    qc = rng.integers(0, 256, size=(B, H, N, 64), dtype=np.uint8)
    kc = rng.integers(0, 256, size=(B, H, N, 64), dtype=np.uint8)
    qs = rng.integers(127, 140, size=(B, H, N, 4), dtype=np.uint8)
    ks = rng.integers(127, 140, size=(B, H, N, 4), dtype=np.uint8)
    v8 = rng.integers(0, 0x7F, size=(B, H, N, 128), dtype=np.uint8)
    sm = float(np.float32(1 / math.sqrt(128)))
    vt = np.zeros((B * H, 128, kq.kq_vt_ld(N)), np.uint8)
    vt[:, :, :N] = v8.reshape(B * H, N, 128).transpose(0, 2, 1)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    o = torch.empty((B, H, N, 128), dtype=torch.float32, device="cuda")
    kq.kq_attn_mxfp4_fwd(dev(qc), dev(qs), dev(kc), dev(ks), dev(vt), 0.01, sm, o)
    torch.cuda.synchronize()
    # the largest |t| these scales allow: 6 * 6 * 2^12 * 2^12 * 128 * sm * log2(e)
    print(f"  |t| bound {36 * 2.0 ** 24 * 128 * sm / math.log(2):.3g}", flush=True)
    assert torch.isfinite(o).all()
