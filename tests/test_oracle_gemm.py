"""Pins for the oracle's quantized projection GEMMs (FP8 W8A8 and MXFP4).

Each pin fixes the result by something other than the oracle's own formula: closed forms
(all-ones, one-hot selection), an int64 route for the exactness claim, a hand-computed
MXFP4 fixture, exact power-of-two scale shifts, and error bounds against the unquantized
float64 product."""
import os

import numpy as np

from oracle import formats as F
from oracle import gemm as G
from oracle import quant as Qz

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
ONE_E4M3 = 0x38        # 1.0 = 2^(7-7) * 1.000
ONE_E2M1 = 0x2         # 1.0


def _codes_e4m3(rng, shape):
    c = rng.integers(0, 256, shape).astype(np.uint8)
    return np.where((c & 0x7F) == 0x7F, c & 0xF0, c).astype(np.uint8)   # no NaN codes


def test_fp8_all_ones_closed_form():
    M, N, K = 3, 5, 96
    a = np.full((M, K), ONE_E4M3, np.uint8)
    b = np.full((N, K), ONE_E4M3, np.uint8)
    c = G.gemm_fp8(a, b, np.float32(0.5), np.float32(0.25))
    assert np.array_equal(c, np.full((M, N), K * 0.125))


def test_fp8_one_hot_rows_select_weight_columns():
    rng = np.random.default_rng(1)
    M, N, K = 7, 6, 64
    perm = rng.permutation(K)[:M]
    a = np.zeros((M, K), np.uint8)
    a[np.arange(M), perm] = ONE_E4M3
    b = _codes_e4m3(rng, (N, K))
    c = G.gemm_fp8(a, b, np.float32(2.0), np.float32(0.5))
    expect = F.e4m3_decode(b)[:, perm].T          # C[m, n] = b[n, perm[m]] * 2 * 0.5
    assert np.array_equal(c, expect)


def test_fp8_exact_by_integer_route():
    """Every E4M3 value is v * 2^-9 with v an integer; the int64 product of those integers,
    scaled by 2^-18, must equal the float64 result bit for bit (the exactness claim)."""
    rng = np.random.default_rng(2)
    a = _codes_e4m3(rng, (9, 640))
    b = _codes_e4m3(rng, (11, 640))
    ai = np.rint(F.e4m3_decode(a) * 512).astype(np.int64)
    bi = np.rint(F.e4m3_decode(b) * 512).astype(np.int64)
    assert np.array_equal(ai.astype(np.float64) / 512, F.e4m3_decode(a))
    exact = (ai @ bi.T).astype(np.float64) * 2.0 ** -18
    assert np.array_equal(G.gemm_fp8(a, b, 1.0, 1.0), exact)


def test_fp8_against_unquantized_product():
    """Quantizing both operands with the calibrated scales keeps the product within the
    E4M3 relative rounding (2^-4 per operand) of the unquantized float64 product."""
    rng = np.random.default_rng(3)
    x = rng.standard_normal((16, 256)).astype(np.float32)
    w = (rng.standard_normal((24, 256)) * 0.05).astype(np.float32)
    sa, ia = Qz.fp8_scales(Qz.amax(x))
    sw, iw = Qz.fp8_scales(Qz.amax(w))
    c = G.gemm_fp8(Qz.fp8_codes(x, ia), Qz.fp8_codes(w, iw), sa, sw)
    ref = x.astype(np.float64) @ w.astype(np.float64).T
    mag = np.abs(x.astype(np.float64)) @ np.abs(w.astype(np.float64)).T
    # 2^-4 relative per normal value, plus the subnormal step of each operand
    bound = mag * (2 * 2.0 ** -4 + 2.0 ** -8) + 256 * 2.0 ** -10 * (float(sa) * 4 * np.abs(w).max() + float(sw) * 4 * np.abs(x).max())
    assert np.all(np.abs(c - ref) <= bound)
    assert np.linalg.norm(c - ref) / np.linalg.norm(ref) < 0.05


def _golden_mxfp4():
    rows = []
    with open(os.path.join(GOLDEN, "mxfp4_gemm_example.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                rows.append(line.split())
    blocks = [r for r in rows if r[0] != "expected"]
    expected = float([r for r in rows if r[0] == "expected"][0][1])
    def pack(hexs):
        nib = [int(ch, 16) for ch in hexs]
        return bytes((nib[2 * i] | (nib[2 * i + 1] << 4)) for i in range(len(nib) // 2))
    a_codes = np.frombuffer(b"".join(pack(r[1]) for r in blocks), np.uint8)[None]
    b_codes = np.frombuffer(b"".join(pack(r[3]) for r in blocks), np.uint8)[None]
    a_sc = np.array([[int(r[2]) for r in blocks]], np.uint8)
    b_sc = np.array([[int(r[4]) for r in blocks]], np.uint8)
    return a_codes, a_sc, b_codes, b_sc, expected


def test_mxfp4_hand_computed_example():
    a, sa, b, sb, expected = _golden_mxfp4()
    assert G.gemm_mxfp4(a, sa, b, sb)[0, 0] == expected


def test_mxfp4_scale_byte_shift_is_exact_power_of_two():
    rng = np.random.default_rng(4)
    a = rng.integers(0, 256, (5, 64)).astype(np.uint8)
    b = rng.integers(0, 256, (7, 64)).astype(np.uint8)
    sa = rng.integers(120, 134, (5, 4)).astype(np.uint8)
    sb = rng.integers(120, 134, (7, 4)).astype(np.uint8)
    c = G.gemm_mxfp4(a, sa, b, sb)
    sa2 = sa.copy()
    sa2[2] += 3
    c2 = G.gemm_mxfp4(a, sa2, b, sb)
    assert np.array_equal(c2[2], c[2] * 8.0)
    assert np.array_equal(np.delete(c2, 2, axis=0), np.delete(c, 2, axis=0))


def test_mxfp4_one_hot_rows_select_weight_columns():
    rng = np.random.default_rng(5)
    M, N, K = 6, 5, 128
    perm = rng.permutation(K)[:M]
    vals = np.zeros((M, K), np.uint8)
    vals[np.arange(M), perm] = ONE_E2M1
    a = (vals[:, 0::2] | (vals[:, 1::2] << 4)).astype(np.uint8)
    sa = np.full((M, K // 32), 127, np.uint8)
    b = rng.integers(0, 256, (N, K // 2)).astype(np.uint8)
    sb = rng.integers(124, 131, (N, K // 32)).astype(np.uint8)
    c = G.gemm_mxfp4(a, sa, b, sb)
    bv = Qz.fp4_unpack(b, sb)
    assert np.array_equal(c, bv[:, perm].T)


def test_mxfp4_against_unquantized_product():
    """Block FP4 of both operands keeps the product within E2M1's relative rounding
    (1/4 of the value per operand, plus half the smallest step of each block)."""
    rng = np.random.default_rng(6)
    x = rng.standard_normal((12, 256)).astype(np.float32)
    w = (rng.standard_normal((20, 256)) * 0.1).astype(np.float32)
    xc, xs, xdq = Qz.fp4_block_quant(x)
    wc, ws, wdq = Qz.fp4_block_quant(w)
    c = G.gemm_mxfp4(xc, xs, wc, ws)
    assert np.array_equal(c, xdq.astype(np.float64) @ wdq.astype(np.float64).T)
    ref = x.astype(np.float64) @ w.astype(np.float64).T
    assert np.linalg.norm(c - ref) / np.linalg.norm(ref) < 0.3
