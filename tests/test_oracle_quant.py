"""Pins for the oracle's calibration, FP8 fake-quant, FP4 block fake-quant and RoPE."""
import math
import os

import numpy as np
import torch

import workloads as W
from oracle import formats as F
from oracle import quant as Qz
from oracle import rope as R

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    out = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                out.append(line.split())
    return out


# ---------------------------------------------------------------- calibration and FP8

def test_amax_is_order_free_max():
    x = W.bits_to_f32(W.random_bits(1, 2, 300, 128, seed=11, outliers=True))
    perm = np.random.default_rng(0).permutation(x.size)
    assert Qz.amax(x) == float(np.max(np.abs(x)))
    assert Qz.amax(x.reshape(-1)[perm]) == Qz.amax(x)
    assert Qz.amax(np.zeros(5, np.float32)) == 0.0


def test_fp8_scale_rule():
    s, inv = Qz.fp8_scales(448.0)
    assert s == 1.0 and inv == 1.0
    s, inv = Qz.fp8_scales(0.0)
    assert s == 1.0 and inv == 1.0
    s, inv = Qz.fp8_scales(3.5)
    assert s.dtype == np.float32 and inv.dtype == np.float32
    assert s == np.float32(3.5 / 448.0) and inv == np.float32(448.0 / 3.5)


def test_fp8_amax_maps_to_max_code():
    x = W.bits_to_f32(W.random_bits(1, 3, 257, 128, seed=5, outliers=True))
    s, inv = Qz.fp8_scales(Qz.amax(x))
    c = Qz.fp8_codes(x, inv)
    assert (c & 0x7F).max() == 0x7E                    # amax lands on 448
    assert np.all(np.abs(Qz.fp8_dequant(c, s)) <= Qz.amax(x) * (1 + 2 ** -20))


def test_fp8_fake_quant_idempotent():
    x = W.bits_to_f32(W.random_bits(2, 2, 129, 128, seed=9, outliers=True))
    s, inv = Qz.fp8_scales(Qz.amax(x))
    c1 = Qz.fp8_codes(x, inv)
    y = Qz.fp8_dequant(c1, s).astype(np.float32)
    c2 = Qz.fp8_codes(y, inv)
    assert np.array_equal(c1, c2)


def test_fp8_codes_match_torch_cast():
    x = W.bits_to_f32(W.random_bits(1, 2, 500, 128, seed=21, outliers=True))
    _, inv = Qz.fp8_scales(Qz.amax(x))
    y = x * inv
    ref = torch.from_numpy(np.clip(y, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8)
    assert np.array_equal(Qz.fp8_codes(x, inv), ref.numpy())


# ---------------------------------------------------------------- FP4 block

def test_fp4_worked_block():
    rows = _rows("fp4_block_example.txt")
    x = np.array([float(r[0]) for r in rows], np.float32)
    codes_want = np.array([int(r[1], 16) for r in rows], np.uint8)
    dq_want = np.array([float(r[2]) for r in rows], np.float64)
    for k, byte in ((0, 127), (-10, 117)):
        xs = (x * np.float32(2.0 ** k)).astype(np.float32)
        codes, scales, dq = Qz.fp4_block_quant(xs[None, :])
        c = np.stack([codes[0] & 0xF, codes[0] >> 4], axis=-1).reshape(-1)
        assert np.array_equal(c, codes_want)
        assert scales[0, 0] == byte
        assert np.array_equal(dq[0].astype(np.float64), dq_want * 2.0 ** k)


def test_fp4_low_nibble_is_even_element():
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = 6.0     # code 7
    x[0, 1] = -0.5    # code 9
    codes, _, _ = Qz.fp4_block_quant(x)
    assert codes[0, 0] == 0x97


def test_fp4_idempotent_and_exact_in_bf16():
    x = W.bits_to_f32(W.random_bits(1, 4, 200, 128, seed=31, outliers=True))
    c1, s1, dq1 = Qz.fp4_block_quant(x)
    c2, s2, dq2 = Qz.fp4_block_quant(dq1)
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2) and np.array_equal(dq1, dq2)
    F.f32_to_bf16_bits_exact(dq1)                       # raises if not representable
    assert np.array_equal(Qz.fp4_unpack(c1, s1), dq1.astype(np.float64))


def test_fp4_scale_equivariance_and_bounds():
    x = W.bits_to_f32(W.random_bits(1, 1, 64, 128, seed=41))
    _, s0, dq0 = Qz.fp4_block_quant(x)
    for k in (-20, -3, 5, 17):
        _, sk, dqk = Qz.fp4_block_quant((x * np.float32(2.0 ** k)).astype(np.float32))
        assert np.array_equal(sk.astype(int), s0.astype(int) + k)
        assert np.array_equal(dqk, (dq0 * np.float32(2.0 ** k)).astype(np.float32))
    blocks = dq0.reshape(-1, 32).astype(np.float64)
    e = s0.reshape(-1).astype(int) - 127
    assert np.all(np.abs(blocks).max(axis=1) <= 6.0 * 2.0 ** e)
    assert np.all(np.abs(blocks).max(axis=1) >= 2.0 ** e)   # amax >= 4 * 2^e rounds to >= 4*2^e


def test_fp4_zero_block_and_tiny_blocks():
    x = np.zeros((2, 64), np.float32)
    x[1, 32:] = np.float32(2.0 ** -130)           # float32 subnormal block
    x[1, 33] = np.float32(-(2.0 ** -131))
    codes, scales, dq = Qz.fp4_block_quant(x)
    assert np.all(codes[0] == 0) and np.all(scales[0] == 0) and np.all(dq[0] == 0)
    assert scales[1, 1] == 0                       # e clamps to -127
    # 2^-130 / 2^-127 = 0.125 -> 0; -2^-131 -> -0
    assert codes[1, 16] == 0x80


# ---------------------------------------------------------------- RoPE

def test_rope_table_closed_form_entries():
    pos = np.array([[0, 0, 0], [1, 0, 0], [0, 1, 0], [0, 0, 3], [1, 47, 63]], np.int32)
    tab = R.table(pos)
    assert tab.shape == (5, 64, 2)
    assert np.all(tab[0, :, 0] == 1.0) and np.all(tab[0, :, 1] == 0.0)
    # axis 0 owns pairs 0..7, axis 1 pairs 8..35, axis 2 pairs 36..63; pair k of an axis
    # has angular frequency 10000^(-2k/d_a)
    assert tab[1, 0, 0] == np.float32(math.cos(1.0)) and tab[1, 0, 1] == np.float32(math.sin(1.0))
    assert np.all(tab[1, 8:, 0] == 1.0)
    w = 10000.0 ** (-2.0 * 3 / 16)
    assert abs(tab[1, 3, 1] - math.sin(w)) < 1e-7
    assert tab[2, 8, 1] == np.float32(math.sin(1.0)) and np.all(tab[2, :8, 0] == 1.0)
    w = 10000.0 ** (-2.0 * 5 / 56)
    assert abs(tab[3, 36 + 5, 0] - math.cos(3 * w)) < 1e-7
    assert abs(tab[4, 8 + 27, 1] - math.sin(47 * 10000.0 ** (-54.0 / 56))) < 1e-7


def test_rope_rotates_counterclockwise_and_text_unchanged():
    pos = np.array([[0, 0, 0], [0, 2, 0]], np.int32)
    tab = R.table(pos)
    x = np.zeros((2, 128), np.float32)
    x[:, 16] = 1.0                                  # pair 8 = first pair of axis 1
    y = R.apply(x, tab)
    assert np.array_equal(y[0], x[0])
    assert y[1, 16] == np.float32(math.cos(2.0)) and y[1, 17] == np.float32(math.sin(2.0))
    q = W.bits_to_f32(W.random_bits(1, 2, 2, 128, seed=3))
    assert np.array_equal(R.apply(q, tab)[..., 0, :], q[..., 0, :])


def test_rope_preserves_pair_norms_and_relative_positions():
    c = W.config(5)
    pos = W.positions(c)[::97]
    tab = R.table(pos)
    x = W.bits_to_f32(W.random_bits(1, 1, len(pos), 128, seed=8))[0, 0]
    y = R.apply(x, tab).astype(np.float64)
    n0 = x[:, 0::2].astype(np.float64) ** 2 + x[:, 1::2].astype(np.float64) ** 2
    n1 = y[:, 0::2] ** 2 + y[:, 1::2] ** 2
    assert np.allclose(n0, n1, rtol=3e-6, atol=1e-30)
    # <R_m a, R_n b> depends only on m - n: shift both positions by the same offset
    a = W.bits_to_f32(W.random_bits(1, 1, 1, 128, seed=12))[0, 0, 0]
    b = W.bits_to_f32(W.random_bits(1, 1, 1, 128, seed=13))[0, 0, 0]
    pm = np.array([[0, 5, 9], [1, 2, 30]], np.int32)
    shift = np.array([1, 11, 7], np.int32)
    t0 = R.table(pm)
    t1 = R.table(pm + shift)
    d0 = float(np.dot(R.apply(a[None], t0[:1])[0].astype(np.float64),
                      R.apply(b[None], t0[1:])[0].astype(np.float64)))
    d1 = float(np.dot(R.apply(a[None], t1[:1])[0].astype(np.float64),
                      R.apply(b[None], t1[1:])[0].astype(np.float64)))
    assert abs(d0 - d1) < 2e-4 * (1 + abs(d0))


def test_workload_positions_follow_token_layout():
    c = W.config(5)
    pos = W.positions(c)
    assert pos.shape == (4608, 3)
    assert np.all(pos[:512] == 0)
    tgt = pos[512:512 + 3072]
    assert np.all(tgt[:, 0] == 0) and tgt[:, 1].max() == 47 and tgt[:, 2].max() == 63
    ctx = pos[512 + 3072:]
    assert np.all(ctx[:, 0] == 1) and ctx[:, 1].max() == 31 and ctx[:, 2].max() == 31
    assert sum(R.AXES) == 128
