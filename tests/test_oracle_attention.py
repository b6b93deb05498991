"""Pins for the oracle's attention (R3) and the end-to-end pipeline.

Independent checks: torch's scaled_dot_product_attention in float64 when the
quantizers are switched off; a case where P's FP8 quantization is lossless;
a from-scratch one-pass (flash-style) schedule with an integer running max;
an int64 route for the exactness of both matrix products; softmax invariants.
"""
import math

import numpy as np
import torch

import workloads as W
from oracle import attention as A
from oracle import formats as F
from oracle import pipeline as P
from oracle import quant as Qz


def rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def _codes(shape, seed, hi=0x7E):
    rng = np.random.default_rng(seed)
    c = rng.integers(0, hi + 1, size=shape).astype(np.uint8)
    sign = rng.integers(0, 2, size=shape).astype(np.uint8) << 7
    return c | sign


# ---------------------------------------------------------------- exactness of the BMMs

def test_bmm_exact_against_int64_route():
    q = _codes((64, 128), 1)
    k = _codes((300, 128), 2)
    q[0] = 0x7E                        # worst case magnitudes: 448 * 448 * 128
    k[0] = 0x7E
    qi = np.rint(F.e4m3_decode(q) * 512).astype(np.int64)      # every E4M3 value is n * 2^-9
    ki = np.rint(F.e4m3_decode(k) * 512).astype(np.int64)
    assert np.array_equal(qi / 512.0, F.e4m3_decode(q))
    exact = (qi @ ki.T).astype(np.float64) / 2.0 ** 18
    assert np.array_equal(F.e4m3_decode(q) @ F.e4m3_decode(k).T, exact)
    # BMM2 at full length with every P code at 448
    n = 8704
    p = np.full((4, n), 0x7E, np.uint8)
    v = _codes((n, 128), 3)
    vi = np.rint(F.e4m3_decode(v) * 512).astype(np.int64)
    pi = np.rint(F.e4m3_decode(p) * 512).astype(np.int64)
    assert np.array_equal(F.e4m3_decode(p) @ F.e4m3_decode(v), (pi @ vi) / 2.0 ** 18)


# ---------------------------------------------------------------- quantizers off

def _pin_unquantized_equals_sdpa(N=200, H=2, seed=5):
    x = [W.bits_to_f32(W.random_bits(1, H, N, 128, seed + t)).astype(np.float64)
         for t in range(3)]
    sm = np.float32(1.0 / math.sqrt(128))
    c1, _ = A.constants(1.0, 1.0, 1.0, sm)
    for h in range(H):
        O, _, _ = A.r3_rows(x[0][0, h], x[1][0, h], x[2][0, h], c1, 1.0 / 448.0,
                            quantize_p=False)
        ref = torch.nn.functional.scaled_dot_product_attention(
            *(torch.from_numpy(t[0, h][None]) for t in x), scale=float(sm))[0].numpy()
        assert rel_l2(O, ref) < 1e-6, rel_l2(O, ref)
        assert np.max(np.abs(O - ref)) < 1e-5


def test_r3_without_quantization_is_softmax_attention():
    _pin_unquantized_equals_sdpa()
    _pin_unquantized_equals_sdpa(N=128, H=1, seed=9)


def _pin_lossless_p_equals_softmax():
    """Integer scores with c1 = 1 make every p = 2^-k exact in E4M3 after the 448 scale,
    so R3 must equal base-2 softmax attention on the dequantized operands exactly."""
    rng = np.random.default_rng(4)
    N, d = 96, 128
    q8 = np.zeros((1, 1, N, d), np.uint8)
    k8 = np.zeros((1, 1, N, d), np.uint8)
    q8[..., 0] = 0x38                                     # q = e_0 (1.0)
    k8[0, 0, :, 0] = F.e4m3_encode(-rng.integers(0, 12, size=N).astype(np.float64))
    v8 = _codes((1, 1, N, d), 8, hi=0x60)
    sm = np.float32(math.log(2.0))                        # fl32(fl32(ln 2) log2 e) == 1
    s_v = np.float32(0.75)
    c1, _ = A.constants(1.0, 1.0, s_v, sm)
    assert c1 == 1.0
    O, M, l = A.attention_r3(q8, k8, v8, 1.0, 1.0, s_v, sm)
    raw = F.e4m3_decode(q8[0, 0]) @ F.e4m3_decode(k8[0, 0]).T
    w = np.exp2(raw - raw.max(axis=1, keepdims=True))
    ref = (w / w.sum(axis=1, keepdims=True)) @ (F.e4m3_decode(v8[0, 0]) * 0.75)
    assert np.max(np.abs(O[0, 0] - ref)) <= 1e-6 * np.max(np.abs(ref))
    assert np.all(M[0, 0] == np.ceil(raw.max(axis=1)))


def test_r3_lossless_p_case():
    _pin_lossless_p_equals_softmax()


# ---------------------------------------------------------------- P quantization, lossy

def _pin_r3_against_torch_fp8_cast():
    """The same definition evaluated with torch's float8_e4m3fn casts for every FP8 step."""
    q, k, v = (W.bits_to_f32(b) for b in W.qkv_bits(1))
    qz = P.quantize_inputs(*W.qkv_bits(1))
    O, M, l = P.attention(qz)

    def t8(x, inv):
        y = torch.from_numpy(np.clip(np.asarray(x, np.float32) * np.float32(inv), -448, 448))
        return y.to(torch.float8_e4m3fn).to(torch.float64)

    sq, iq = Qz.fp8_scales(np.max(np.abs(q)))
    sk, ik = Qz.fp8_scales(np.max(np.abs(k)))
    sv, iv = Qz.fp8_scales(np.max(np.abs(v)))
    c1 = np.float32(float(sq) * float(sk) * float(np.float32(1 / math.sqrt(128))) / math.log(2))
    for h in range(q.shape[1]):
        raw = t8(q[0, h], iq) @ t8(k[0, h], ik).T
        t = (raw * float(c1)).to(torch.float32).to(torch.float64)
        m = torch.ceil(t.max(dim=1, keepdim=True).values)
        p = torch.exp2(t - m).to(torch.float32)
        lsum = p.to(torch.float64).sum(dim=1).to(torch.float32)
        pq = (p * 448.0).clamp(max=448).to(torch.float8_e4m3fn).to(torch.float64)
        ref = (pq @ t8(v[0, h], iv)) * float(np.float32(float(sv) / 448.0))
        ref = (ref / lsum.to(torch.float64)[:, None]).to(torch.float32).numpy()
        assert rel_l2(O[0, h], ref) < 1e-6, rel_l2(O[0, h], ref)


def test_r3_matches_torch_cast_evaluation():
    _pin_r3_against_torch_fp8_cast()


def _pin_softmax_invariants():
    qz = P.quantize_inputs(*W.qkv_bits(1))
    q8, k8 = qz.codes["q"], qz.codes["k"]
    c1, _ = A.constants(qz.scale["q"][0], qz.scale["k"][0], qz.scale["v"][0],
                        np.float32(1 / math.sqrt(128)))
    for h in range(q8.shape[1]):
        raw = F.e4m3_decode(q8[0, h]) @ F.e4m3_decode(k8[0, h]).T
        t = F.fl32(raw * float(c1)).astype(np.float64)
        O, M, l = A.r3_rows(F.e4m3_decode(q8[0, h]), F.e4m3_decode(k8[0, h]),
                            F.e4m3_decode(qz.codes["v"][0, h]), c1, 1.0)
        assert np.all(M == np.ceil(t.max(axis=1)))
        p = np.exp2(t - M[:, None])
        pmax = p.max(axis=1)
        assert np.all(pmax > 0.5) and np.all(pmax <= 1.0)
        assert np.allclose((p / l[:, None].astype(np.float64)).sum(axis=1), 1.0, atol=1e-6)


def test_r3_softmax_invariants():
    _pin_softmax_invariants()


# ---------------------------------------------------------------- one-pass schedule

def _one_pass(q8, k8, v8, s_q, s_k, s_v, sm, tile):
    """Flash-style schedule written independently: keys in tiles, integer running offset,
    P quantized per tile against the current offset, power-of-two rescale of acc and l."""
    Qv = F.e4m3_decode(q8)
    Kv = F.e4m3_decode(k8)
    Vv = F.e4m3_decode(v8)
    c1 = np.float32(float(np.float32(s_q)) * float(np.float32(s_k)) * float(np.float32(sm))
                    / math.log(2))
    R, d = Qv.shape
    m = np.full(R, -np.inf)
    l = np.zeros(R)
    acc = np.zeros((R, d))
    for j0 in range(0, Kv.shape[0], tile):
        t = (Qv @ Kv[j0:j0 + tile].T * float(c1)).astype(np.float32).astype(np.float64)
        m_new = np.maximum(m, np.ceil(t.max(axis=1)))
        alpha = np.exp2(m - m_new)
        p = np.exp2(t - m_new[:, None]).astype(np.float32)
        l = l * alpha + p.astype(np.float64).sum(axis=1)
        code = torch.from_numpy((p * np.float32(448)).astype(np.float32)).to(torch.float8_e4m3fn)
        acc = acc * alpha[:, None] + code.to(torch.float64).numpy() @ Vv[j0:j0 + tile]
        m = m_new
    return acc * (float(np.float32(s_v)) / 448.0) / l[:, None]


def test_r3_is_what_a_one_pass_schedule_computes():
    for cfg, n_heads, tile in ((1, 2, 64), (2, 2, 128)):
        bits = [b[:, :n_heads] for b in W.qkv_bits(cfg)]
        qz = P.quantize_inputs(*bits)
        O, _, _ = P.attention(qz)
        for h in range(n_heads):
            F1 = _one_pass(qz.codes["q"][0, h], qz.codes["k"][0, h], qz.codes["v"][0, h],
                           qz.scale["q"][0], qz.scale["k"][0], qz.scale["v"][0],
                           np.float32(1 / math.sqrt(128)), tile)
            assert rel_l2(F1, O[0, h]) < 1e-4, (cfg, h, rel_l2(F1, O[0, h]))


# ---------------------------------------------------------------- end to end

def test_pipeline_tiny_against_unquantized_fp64():
    qb, kb, vb = W.qkv_bits(1)
    qz = P.quantize_inputs(qb, kb, vb)
    O, _, _ = P.attention(qz)
    ref = A.attention_fp64(W.bits_to_f32(qb), W.bits_to_f32(kb), W.bits_to_f32(vb),
                           1 / math.sqrt(128))
    err = rel_l2(O, ref)
    assert 1e-3 < err < 0.1, err           # FP8 Q/K/V/P noise, no outliers: a few percent
    O1, amax_p = A.attention_r1(qz.codes["q"], qz.codes["k"], qz.codes["v"], qz.scale["q"][0],
                                qz.scale["k"][0], qz.scale["v"][0],
                                np.float32(1 / math.sqrt(128)))
    assert 0 < amax_p <= 1.0
    assert rel_l2(O1, ref) < 0.1


def _pin_r1_closed_form():
    """R1 on integer scores 0 (n_a keys) and -1 (n_b keys) with c1 = 1: p is 1 or 1/2, the
    row sum l = n_a + n_b / 2, P = 1/l or 1/(2l), the calibrated amax_P = 1/l, and the FP8
    codes of P / s_P are exactly 448 and 224, so O = (sum_a v + sum_b v / 2) s_V / l."""
    rng = np.random.default_rng(12)
    N, d = 80, 128
    q8 = np.zeros((1, 1, N, d), np.uint8)
    k8 = np.zeros((1, 1, N, d), np.uint8)
    q8[..., 0] = 0x38                                     # q = e_0 (1.0)
    grp_b = rng.random(N) < 0.4
    k8[0, 0, grp_b, 0] = 0xB8                             # -1.0: score -1
    v8 = _codes((1, 1, N, d), 13, hi=0x60)
    sm, s_v = np.float32(math.log(2.0)), np.float32(0.5)
    O, amax_p = A.attention_r1(q8, k8, v8, 1.0, 1.0, s_v, sm)
    n_a, n_b = int(np.sum(~grp_b)), int(np.sum(grp_b))
    l = n_a + 0.5 * n_b
    assert amax_p == float(np.float32(1.0 / l))
    vv = F.e4m3_decode(v8[0, 0]) * float(s_v)
    ref = (vv[~grp_b].sum(axis=0) + 0.5 * vv[grp_b].sum(axis=0)) / l
    assert np.allclose(O[0, 0], np.broadcast_to(ref, O[0, 0].shape), rtol=1e-6, atol=0)
    # the same rows evaluated alone with the same static amax_P
    Os, _ = A.attention_r1(q8, k8, v8, 1.0, 1.0, s_v, sm, amax_p=amax_p, rows=np.array([3, 79]))
    assert np.array_equal(Os[0, 0], O[0, 0, [3, 79]])


def test_r1_closed_form():
    _pin_r1_closed_form()


def test_pipeline_sampled_rows_equal_full_rows():
    qz = P.quantize_inputs(*W.qkv_bits(1))
    O, M, l = P.attention(qz)
    rows = np.array([0, 7, 63, 64, 200, 255])
    Os, Ms, ls = P.attention(qz, rows=rows)
    assert np.array_equal(Os, O[:, :, rows]) and np.array_equal(ls, l[:, :, rows])


def test_pipeline_fp4_rope_small():
    c = W.config(5)
    pos = W.positions(c)[:300]
    bits = [W.random_bits(1, 2, 300, 128, seed=70 + t, outliers=True) for t in range(3)]
    qz = P.quantize_inputs(*bits, mode="fp4", positions=pos)
    for n in "qkv":
        F.f32_to_bf16_bits_exact(qz.x[n])          # FP8 quantizer input is the FP4 dequant
        assert qz.amax[n] == float(np.max(np.abs(qz.fp4[n][2])))
    O, _, _ = P.attention(qz)
    assert np.all(np.isfinite(O))


# ---------------------------------------------------------------- native MXFP4 BMM1 variant

_E2M1_MAGS = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])   # OCP MX E2M1, codes 0-7


def _fp4_operands(shape, seed, lo=119, hi=133):
    """Random E2M1 elements (all 16 codes) packed by hand (even element in the low nibble),
    E8M0 scales in [lo, hi], and their values computed here from the OCP table: every value
    E2M1 * 2^e with -8 <= e <= 6 is a multiple of 2^-9 below 448, i.e. exact in E4M3."""
    B, H, N, d = shape
    rng = np.random.default_rng(seed)
    nib = rng.integers(0, 16, size=(B, H, N, d), dtype=np.uint8)
    scales = rng.integers(lo, hi + 1, size=(B, H, N, d // 32), dtype=np.uint8)
    sign = np.where(nib & 8, -1.0, 1.0)
    values = sign * _E2M1_MAGS[nib & 7] * np.repeat(2.0 ** (scales.astype(np.float64) - 127),
                                                     32, axis=-1)
    codes = (nib[..., 0::2] | (nib[..., 1::2] << 4)).astype(np.uint8)
    return codes, scales, values


def _pin_r3_mxfp4_equals_fp8_r3():
    shape = (1, 2, 96, 128)
    qc, qs, qv = _fp4_operands(shape, 1)
    kc, ks, kv = _fp4_operands(shape, 2)
    v8 = _codes(shape, 3)
    q8, k8 = F.e4m3_encode(qv), F.e4m3_encode(kv)
    assert np.array_equal(F.e4m3_decode(q8), qv) and np.array_equal(F.e4m3_decode(k8), kv)
    sv, sm = np.float32(0.02), np.float32(1 / math.sqrt(128))
    o4, m4, l4 = A.attention_r3_mxfp4(qc, qs, kc, ks, v8, sv, sm)
    o8, m8, l8 = A.attention_r3(q8, k8, v8, 1.0, 1.0, sv, sm)
    assert np.array_equal(o4, o8) and np.array_equal(m4, m8) and np.array_equal(l4, l8)


def test_r3_mxfp4_equals_fp8_r3_when_fp4_values_are_e4m3_exact():
    """When every FP4 value is an exact E4M3 value, BMM1 on the FP4 operands and BMM1 on their
    E4M3 codes with unit per-tensor scales are the same products: the MXFP4 variant must equal
    the (independently pinned) FP8 R3 bit for bit."""
    _pin_r3_mxfp4_equals_fp8_r3()


def test_r3_mxfp4_rows_subset_and_real_quantizer_output():
    """Sampled rows equal the full evaluation, and on the FP4 quantizer's own output the
    result tracks unquantized float64 attention of the dequantized inputs."""
    bits = [W.random_bits(1, 1, 200, 128, seed=90 + t, outliers=True) for t in range(3)]
    x = [W.bits_to_f32(b) for b in bits]
    (qc, qs, qd), (kc, ks, kd) = Qz.fp4_block_quant(x[0]), Qz.fp4_block_quant(x[1])
    sv, iv = Qz.fp8_scales(Qz.amax(x[2]))
    v8 = Qz.fp8_codes(x[2], iv)
    sm = np.float32(1 / math.sqrt(128))
    O, _, _ = A.attention_r3_mxfp4(qc, qs, kc, ks, v8, sv, sm)
    rows = np.array([0, 7, 199])
    Os, _, _ = A.attention_r3_mxfp4(qc, qs, kc, ks, v8, sv, sm, rows=rows)
    assert np.array_equal(Os, O[:, :, rows])
    ref = A.attention_fp64(qd, kd, F.e4m3_decode(v8) * float(sv), sm)
    assert rel_l2(O, ref) < 3e-2
