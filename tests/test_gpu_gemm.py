"""GPU parity of the quantized projection GEMMs (kq_gemm_fp8, kq_gemm_mxfp4 and their bf16-output
forms) against the oracle.

Each side quantizes the same seeded bf16 activations and weights with its own code (the HIP
quantizers on the device, the oracle's on the CPU), the codes must agree bit for bit, and
the products must agree within the bound the arithmetic fixes:

  the oracle's C is exact (float64; see oracle/gemm.py).  The device sums each MFMA's products
  and adds them to a float32 accumulator, so with L1 = scale * sum_k |a_k b_k|:
    |C_gpu - C| <= (K * 2^-24 + 2^-23) * L1              (float32 additions, final scaling)
  plus, for FP8, the matrix core's product truncation: products of E4M3 operands are summed in
  groups of 8 consecutive k after truncation toward zero to a quantum of
  2^(floor(log2 max|p|) - 13) of the group's largest product, at most 2^-10 * L1 in total.
An E2M1 product has at most 4 significant bits and the products of one group of 8 share their
32-block's scale, so a group sums to a multiple of 2^-2 below 2^9 times that scale, exact at
any truncation quantum as fine as the one above: the FP4 path has no truncation term.

Sizes: small shapes with ragged M and N tails (several 256 x 256 tiles, one to a few k-steps)
run against the full oracle product; the two Kontext projection shapes (M = 8704 tokens,
K = 3072, N = 9216 and 3072) are compared on sampled rows and columns, including both ends of
every tile edge they cross.  Cases whose every product and partial sum is exact in float32
must match bit for bit.

bf16 output: the float32 result rounded once to nearest even.  Rounding is monotone, so each
element must lie between the bf16 roundings of (exact - bound) and (exact + bound), equal the
bf16 rounding of the exact value where the float32 result is exact, and equal torch's bf16
cast of the float32 entry point's result on the same inputs.
"""
import numpy as np
import pytest
import torch

import precision_quantized_attention_amd as kq
import workloads as W
from kq_testutil import to_dev
from oracle import gemm as OG
from oracle import quant as Qz

pytestmark = pytest.mark.gpu

FP8_TRUNC = 2.0 ** -10


def _bound(L1, K, fp8: bool):
    return (K * 2.0 ** -24 + 2.0 ** -23 + (FP8_TRUNC if fp8 else 0.0)) * L1


# ------------------------------------------------------------------ device pipelines

def _gpu_fp8(a_bits, w_bits):
    """HIP path: amax calibration, scale rule, E4M3 quantization, GEMM.  Returns codes and C."""
    a, w = to_dev(a_bits), to_dev(w_bits)
    out = []
    for x in (a, w):
        am = torch.zeros(1, dtype=torch.float32, device="cuda")
        kq.kq_amax_calibrate(x, am)
        s, inv = kq.kq_fp8_scales_from_amax(float(am.item()))
        y = torch.empty(x.shape, dtype=torch.uint8, device="cuda")
        kq.kq_quantize_fp8_tensor(x, inv, y)
        out.append((y, s))
    (a8, sa), (w8, sw) = out
    c = torch.empty((a.shape[0], w.shape[0]), dtype=torch.float32, device="cuda")
    kq.kq_gemm_fp8(a8, w8, sa, sw, c)
    return a8, sa, w8, sw, c


def _gpu_fp4(a_bits, w_bits):
    a, w = to_dev(a_bits), to_dev(w_bits)
    out = []
    for x in (a, w):
        rows, K = x.shape
        codes = torch.empty((rows, K // 2), dtype=torch.uint8, device="cuda")
        scales = torch.empty((rows, K // 32), dtype=torch.uint8, device="cuda")
        kq.kq_quantize_fp4_block(x.view(-1, 128), codes.view(-1, 64), scales.view(-1, 4))
        out.append((codes, scales))
    (ac, asc), (wc, wsc) = out
    c = torch.empty((a.shape[0], w.shape[0]), dtype=torch.float32, device="cuda")
    kq.kq_gemm_mxfp4(ac, asc, wc, wsc, c)
    return ac, asc, wc, wsc, c


# ------------------------------------------------------------------ oracle side

def _oracle_fp8(a_bits, w_bits, a_amax=None, w_amax=None):
    """Oracle codes, scales, exact C and the L1 magnitudes of its terms."""
    af, wf = W.bits_to_f32(a_bits), W.bits_to_f32(w_bits)
    sa, ia = Qz.fp8_scales(Qz.amax(af) if a_amax is None else a_amax)
    sw, iw = Qz.fp8_scales(Qz.amax(wf) if w_amax is None else w_amax)
    a8, w8 = Qz.fp8_codes(af, ia), Qz.fp8_codes(wf, iw)
    c = OG.gemm_fp8(a8, w8, sa, sw)
    L1 = OG.gemm_fp8(a8 & 0x7F, w8 & 0x7F, sa, sw)          # sign bits cleared: sum |a_k b_k|
    return a8, sa, w8, sw, c, L1


def _oracle_fp4(a_bits, w_bits):
    af, wf = W.bits_to_f32(a_bits), W.bits_to_f32(w_bits)
    ac, asc, _ = Qz.fp4_block_quant(af)
    wc, wsc, _ = Qz.fp4_block_quant(wf)
    c = OG.gemm_mxfp4(ac, asc, wc, wsc)
    L1 = OG.gemm_mxfp4(ac & 0x77, asc, wc & 0x77, wsc)
    return ac, asc, wc, wsc, c, L1


def _check_close(c_gpu, c, L1, K, fp8, what):
    err = np.abs(np.asarray(c_gpu, np.float64) - c)
    bound = _bound(L1, K, fp8)
    worst = np.unravel_index(np.argmax(err - bound), err.shape)
    assert np.all(err <= bound), (what, worst, err[worst], bound[worst])
    nrm = np.linalg.norm(c)
    if nrm > 0:
        assert np.linalg.norm(np.asarray(c_gpu, np.float64) - c) / nrm < 2e-3, what


# ------------------------------------------------------------------ small shapes, full product

SMALL = [(300, 260, 192), (520, 516, 384), (1, 4, 128), (257, 8, 64), (64, 256, 1024),
         (513, 772, 256)]


@pytest.mark.parametrize("M,N,K", [s for s in SMALL if s[2] % 64 == 0])
def test_fp8_gemm_matches_oracle(M, N, K):
    print(f"gemm fp8 {M}x{N}x{K}", flush=True)
    a_bits, w_bits = W.gemm_bits(M, N, K, seed=11 + M + N + K)
    a8, sa, w8, sw, c = _gpu_fp8(a_bits, w_bits)
    oa8, osa, ow8, osw, oc, L1 = _oracle_fp8(a_bits, w_bits)
    assert np.array_equal(a8.cpu().numpy(), oa8) and np.array_equal(w8.cpu().numpy(), ow8)
    assert np.float32(sa) == osa and np.float32(sw) == osw
    _check_close(c.cpu().numpy(), oc, L1, K, True, (M, N, K))


@pytest.mark.parametrize("M,N,K", [s for s in SMALL if s[2] % 128 == 0])
def test_mxfp4_gemm_matches_oracle(M, N, K):
    print(f"gemm mxfp4 {M}x{N}x{K}", flush=True)
    a_bits, w_bits = W.gemm_bits(M, N, K, seed=23 + M + N + K)
    ac, asc, wc, wsc, c = _gpu_fp4(a_bits, w_bits)
    oac, oasc, owc, owsc, oc, L1 = _oracle_fp4(a_bits, w_bits)
    assert np.array_equal(ac.cpu().numpy(), oac) and np.array_equal(asc.cpu().numpy(), oasc)
    assert np.array_equal(wc.cpu().numpy(), owc) and np.array_equal(wsc.cpu().numpy(), owsc)
    _check_close(c.cpu().numpy(), oc, L1, K, False, (M, N, K))


# ------------------------------------------------------------------ exact cases, bit for bit

# E4M3 codes of 0, +-0.5, +-1, +-2 (bias 7: 0.5 = 2^-1 -> exponent field 6, and so on)
_SMALL_E4M3 = np.array([0x00, 0x30, 0x38, 0x40, 0xB0, 0xB8, 0xC0], np.uint8)


@pytest.mark.parametrize("M,N,K", [(300, 260, 192), (33, 516, 1024)])
def test_fp8_gemm_exact_on_small_values(M, N, K):
    """Products are multiples of 1/4 up to 4 and sums stay below 2^13: exact in float32 and
    below the truncation quantum, so the device must reproduce the oracle exactly."""
    print(f"gemm fp8 exact {M}x{N}x{K}", flush=True)
    rng = np.random.default_rng(M * N + K)
    a8 = rng.choice(_SMALL_E4M3, size=(M, K))
    w8 = rng.choice(_SMALL_E4M3, size=(N, K))
    c = torch.empty((M, N), dtype=torch.float32, device="cuda")
    kq.kq_gemm_fp8(torch.from_numpy(a8).cuda(), torch.from_numpy(w8).cuda(), 1.0, 1.0, c)
    assert np.array_equal(c.cpu().numpy().astype(np.float64), OG.gemm_fp8(a8, w8, 1.0, 1.0))


@pytest.mark.parametrize("M,N,K", [(300, 260, 256), (70, 516, 512)])
def test_mxfp4_gemm_exact_on_all_codes(M, N, K):
    """Every E2M1 code (both zeros included) with block scales 2^-1 .. 2^1: products are
    multiples of 2^-4 below 144 and sums stay far inside float32's 24 bits."""
    print(f"gemm mxfp4 exact {M}x{N}x{K}", flush=True)
    rng = np.random.default_rng(M + N * K)
    ac = rng.integers(0, 256, size=(M, K // 2), dtype=np.uint8)
    wc = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    asc = rng.integers(126, 129, size=(M, K // 32), dtype=np.uint8)
    wsc = rng.integers(126, 129, size=(N, K // 32), dtype=np.uint8)
    c = torch.empty((M, N), dtype=torch.float32, device="cuda")
    dev = [torch.from_numpy(x).cuda() for x in (ac, asc, wc, wsc)]
    kq.kq_gemm_mxfp4(*dev, c)
    assert np.array_equal(c.cpu().numpy().astype(np.float64), OG.gemm_mxfp4(ac, asc, wc, wsc))


def test_mxfp4_gemm_extreme_block_scales():
    """E8M0 scales at the ends of their range in different blocks of one row: each block's
    products carry their own power of two into the float32 accumulator."""
    print("gemm mxfp4 extreme scales", flush=True)
    rng = np.random.default_rng(5)
    M, N, K = 40, 36, 256
    ac = rng.integers(0, 256, size=(M, K // 2), dtype=np.uint8)
    wc = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    asc = rng.choice(np.array([60, 90, 127, 150, 180], np.uint8), size=(M, K // 32))
    wsc = rng.choice(np.array([70, 100, 127, 140, 170], np.uint8), size=(N, K // 32))
    c = torch.empty((M, N), dtype=torch.float32, device="cuda")
    kq.kq_gemm_mxfp4(*[torch.from_numpy(x).cuda() for x in (ac, asc, wc, wsc)], c)
    oc = OG.gemm_mxfp4(ac, asc, wc, wsc)
    L1 = OG.gemm_mxfp4(ac & 0x77, asc, wc & 0x77, wsc)
    _check_close(c.cpu().numpy(), oc, L1, K, False, "extreme scales")


# ------------------------------------------------------------------ Kontext shapes, sampled

def _sample(n, seed, k=40):
    fixed = [0, 1, 31, 32, 63, 64, 127, 128, 255, 256, 257, n // 2, n - 257, n - 256, n - 1]
    rnd = np.random.default_rng(seed).choice(n, size=k, replace=False)
    return np.unique(np.clip(np.concatenate([fixed, rnd]), 0, n - 1))


@pytest.mark.parametrize("shape", W.GEMM_SHAPES, ids=lambda s: s.name)
@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
def test_gemm_kontext_shapes_sampled(shape, fmt):
    M, N, K = shape.M, shape.N, shape.K
    print(f"gemm {fmt} {shape.name} {M}x{N}x{K}", flush=True)
    seed = 100 + N
    a_bits, w_bits = W.gemm_bits(M, N, K, seed)
    rows, cols = _sample(M, seed), _sample(N, seed + 1)
    if fmt == "fp8":
        a8, sa, w8, sw, c = _gpu_fp8(a_bits, w_bits)
        a_amax = Qz.amax(W.bits_to_f32(a_bits))
        w_amax = Qz.amax(W.bits_to_f32(w_bits))
        oa8, osa, ow8, osw, oc, L1 = _oracle_fp8(a_bits[rows], w_bits[cols], a_amax, w_amax)
        assert np.array_equal(a8[torch.from_numpy(rows).cuda()].cpu().numpy(), oa8)
        assert np.array_equal(w8[torch.from_numpy(cols).cuda()].cpu().numpy(), ow8)
        assert np.float32(sa) == osa and np.float32(sw) == osw
    else:
        ac, asc, wc, wsc, c = _gpu_fp4(a_bits, w_bits)
        oac, oasc, owc, owsc, oc, L1 = _oracle_fp4(a_bits[rows], w_bits[cols])
        r, q = torch.from_numpy(rows).cuda(), torch.from_numpy(cols).cuda()
        assert np.array_equal(ac[r].cpu().numpy(), oac) and np.array_equal(asc[r].cpu().numpy(), oasc)
        assert np.array_equal(wc[q].cpu().numpy(), owc) and np.array_equal(wsc[q].cpu().numpy(), owsc)
    got = c[torch.from_numpy(rows).cuda()][:, torch.from_numpy(cols).cuda()].cpu().numpy()
    _check_close(got, oc, L1, K, fmt == "fp8", (fmt, shape.name))
    assert torch.isfinite(c).all().item()


def test_fp8_gemm_output_beyond_2_31_elements():
    """M = 262144 tokens (30 Kontext sequences), N = 9216, K = 3072: C holds 2.4e9 float32
    values (9.7 GB), so output offsets pass 32 bits; sampled rows on both sides of the row
    where m * N crosses 2^31 and at every tile edge are checked against the exact oracle."""
    M, N, K = 262144, 9216, 3072
    assert M * N > 2 ** 31
    print(f"gemm fp8 large {M}x{N}x{K}", flush=True)
    rng = np.random.default_rng(2024)
    a8 = rng.integers(0, 256, size=(M, K), dtype=np.uint8)
    w8 = rng.integers(0, 256, size=(N, K), dtype=np.uint8)
    a8[(a8 & 0x7F) == 0x7F] -= 1                   # no NaN codes
    w8[(w8 & 0x7F) == 0x7F] -= 1
    sa, sw = 2.0 ** -6, 2.0 ** -5
    c = torch.empty((M, N), dtype=torch.float32, device="cuda")
    kq.kq_gemm_fp8(torch.from_numpy(a8).cuda(), torch.from_numpy(w8).cuda(), sa, sw, c)
    cross = (2 ** 31) // N
    rows = np.unique(np.concatenate([_sample(M, 7), [cross - 1, cross, cross + 1, cross + 255]]))
    cols = _sample(N, 8)
    got = c[torch.from_numpy(rows).cuda()][:, torch.from_numpy(cols).cuda()].cpu().numpy()
    oc = OG.gemm_fp8(a8[rows], w8[cols], sa, sw)
    L1 = OG.gemm_fp8(a8[rows] & 0x7F, w8[cols] & 0x7F, sa, sw)
    _check_close(got, oc, L1, K, True, "fp8 large")
    del c
    torch.cuda.empty_cache()


# ------------------------------------------------------------------ bf16 output

def _bf16_round(x64):
    """float64 -> bf16 (one round to nearest even) -> float64."""
    return torch.from_numpy(np.asarray(x64, np.float64)).to(torch.bfloat16).to(torch.float64).numpy()


def _check_bf16(c_bf16, c, L1, K, fp8, what):
    """The device rounds its float32 result once to bf16, and rounding is monotone, so every
    element lies between the bf16 roundings of the exact value minus and plus the float32
    bound."""
    got = c_bf16.to(torch.float64).cpu().numpy() if isinstance(c_bf16, torch.Tensor) else c_bf16
    b = _bound(L1, K, fp8)
    lo, hi = _bf16_round(c - b), _bf16_round(c + b)
    bad = (got < lo) | (got > hi)
    assert not bad.any(), (what, np.argwhere(bad)[:3])


@pytest.mark.parametrize("M,N,K", [(300, 260, 192), (513, 772, 256), (257, 8, 64)])
def test_fp8_gemm_bf16_out_matches_oracle(M, N, K):
    print(f"gemm fp8 bf16-out {M}x{N}x{K}", flush=True)
    a_bits, w_bits = W.gemm_bits(M, N, K, seed=31 + M + N + K)
    a8, sa, w8, sw, c32 = _gpu_fp8(a_bits, w_bits)
    _, _, _, _, oc, L1 = _oracle_fp8(a_bits, w_bits)
    c16 = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    kq.kq_gemm_fp8_bf16(a8, w8, sa, sw, c16)
    torch.cuda.synchronize()
    _check_bf16(c16, oc, L1, K, True, (M, N, K))
    # the same kernel's float32 result, rounded by torch: identical bits
    assert torch.equal(c16, c32.to(torch.bfloat16))


@pytest.mark.parametrize("M,N,K", [(300, 260, 256), (513, 772, 256)])
def test_mxfp4_gemm_bf16_out_matches_oracle(M, N, K):
    print(f"gemm mxfp4 bf16-out {M}x{N}x{K}", flush=True)
    a_bits, w_bits = W.gemm_bits(M, N, K, seed=41 + M + N + K)
    ac, asc, wc, wsc, c32 = _gpu_fp4(a_bits, w_bits)
    _, _, _, _, oc, L1 = _oracle_fp4(a_bits, w_bits)
    c16 = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    kq.kq_gemm_mxfp4_bf16(ac, asc, wc, wsc, c16)
    torch.cuda.synchronize()
    _check_bf16(c16, oc, L1, K, False, (M, N, K))
    assert torch.equal(c16, c32.to(torch.bfloat16))


def test_gemm_bf16_out_exact_cases_round_once():
    """Where every partial sum is exact in float32, the bf16 output is the exact value rounded
    once to nearest even."""
    print("gemm bf16-out exact", flush=True)
    rng = np.random.default_rng(9)
    M, N, K = 300, 260, 192
    a8 = rng.choice(_SMALL_E4M3, size=(M, K))
    w8 = rng.choice(_SMALL_E4M3, size=(N, K))
    c16 = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    kq.kq_gemm_fp8_bf16(torch.from_numpy(a8).cuda(), torch.from_numpy(w8).cuda(), 1.0, 3.0, c16)
    exact = OG.gemm_fp8(a8, w8, 1.0, 3.0)
    assert np.array_equal(c16.to(torch.float64).cpu().numpy(), _bf16_round(exact))
    M, N, K = 70, 516, 512
    ac = rng.integers(0, 256, size=(M, K // 2), dtype=np.uint8)
    wc = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    asc = rng.integers(126, 129, size=(M, K // 32), dtype=np.uint8)
    wsc = rng.integers(126, 129, size=(N, K // 32), dtype=np.uint8)
    c16 = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    kq.kq_gemm_mxfp4_bf16(*[torch.from_numpy(x).cuda() for x in (ac, asc, wc, wsc)], c16)
    assert np.array_equal(c16.to(torch.float64).cpu().numpy(),
                          _bf16_round(OG.gemm_mxfp4(ac, asc, wc, wsc)))


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
def test_gemm_bf16_out_kontext_qkv_sampled(fmt):
    shape = W.GEMM_SHAPES[0]
    M, N, K = shape.M, shape.N, shape.K
    print(f"gemm {fmt} bf16-out {shape.name}", flush=True)
    seed = 200 + N
    a_bits, w_bits = W.gemm_bits(M, N, K, seed)
    rows, cols = _sample(M, seed), _sample(N, seed + 1)
    r, q = torch.from_numpy(rows).cuda(), torch.from_numpy(cols).cuda()
    c16 = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    if fmt == "fp8":
        a8, sa, w8, sw, _ = _gpu_fp8(a_bits, w_bits)
        kq.kq_gemm_fp8_bf16(a8, w8, sa, sw, c16)
        _, _, _, _, oc, L1 = _oracle_fp8(a_bits[rows], w_bits[cols],
                                         Qz.amax(W.bits_to_f32(a_bits)),
                                         Qz.amax(W.bits_to_f32(w_bits)))
    else:
        ac, asc, wc, wsc, _ = _gpu_fp4(a_bits, w_bits)
        kq.kq_gemm_mxfp4_bf16(ac, asc, wc, wsc, c16)
        _, _, _, _, oc, L1 = _oracle_fp4(a_bits[rows], w_bits[cols])
    _check_bf16(c16[r][:, q], oc, L1, K, fmt == "fp8", (fmt, "bf16", shape.name))
    assert torch.isfinite(c16.float()).all().item()


def test_gemm_overwrites_output_and_is_deterministic():
    """C is fully overwritten (no accumulation into prior contents) and two runs agree bit
    for bit."""
    print("gemm overwrite/determinism", flush=True)
    a_bits, w_bits = W.gemm_bits(520, 516, 384, seed=3)
    a8, sa, w8, sw, c1 = _gpu_fp8(a_bits, w_bits)
    c2 = torch.full_like(c1, float("nan"))
    kq.kq_gemm_fp8(a8, w8, sa, sw, c2)
    assert torch.equal(c1, c2)
