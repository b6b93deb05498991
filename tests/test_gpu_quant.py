"""GPU parity of the calibration and quantization kernels: bit-exact against the oracle."""
import numpy as np
import pytest
import torch

import precision_quantized_attention_amd as kq
import workloads as W
from kq_testutil import all_finite_bf16_rows, to_dev
from oracle import formats as F
from oracle import pipeline as OP
from oracle import quant as Qz
from oracle import rope as R

pytestmark = pytest.mark.gpu


def _amax_gpu(x):
    a = torch.zeros(1, dtype=torch.float32, device="cuda")
    kq.kq_amax_calibrate(x, a)
    return float(a.item())


def _split_codes(packed):
    packed = np.asarray(packed, np.uint8)
    return np.stack([packed & 0xF, packed >> 4], axis=-1).reshape(packed.shape[:-1] + (-1,))


# ---------------------------------------------------------------- amax

@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_amax_matches_oracle(cfg):
    print(f"amax cfg{cfg}", flush=True)
    for bits in W.qkv_bits(cfg):
        assert _amax_gpu(to_dev(bits)) == Qz.amax(W.bits_to_f32(bits))


def test_amax_running_max_tail_and_every_bf16():
    bits = all_finite_bf16_rows()
    x = to_dev(bits)
    assert _amax_gpu(x) == Qz.amax(W.bits_to_f32(bits))
    a = torch.zeros(1, dtype=torch.float32, device="cuda")
    small = to_dev(W.random_bits(1, 1, 3, 333, seed=2))              # 999 elements: a tail
    big = to_dev(W.random_bits(1, 1, 7, 128, seed=3, scale=50.0))
    kq.kq_amax_calibrate(big, a)
    kq.kq_amax_calibrate(small, a)
    ref = max(Qz.amax(W.bits_to_f32(W.random_bits(1, 1, 3, 333, seed=2))),
              Qz.amax(W.bits_to_f32(W.random_bits(1, 1, 7, 128, seed=3, scale=50.0))))
    assert float(a.item()) == ref
    assert _amax_gpu(to_dev(W.random_bits(1, 1, 3, 333, seed=2))) == Qz.amax(
        W.bits_to_f32(W.random_bits(1, 1, 3, 333, seed=2)))


# ---------------------------------------------------------------- FP8

@pytest.mark.parametrize("inv", [1.0, 3.7, 0.013, 448.0 / 3.0, 1e-3, 2.0 ** -7, 2.0 ** 20])
def test_fp8_every_bf16(inv):
    bits = all_finite_bf16_rows()
    y = torch.empty(bits.shape, dtype=torch.uint8, device="cuda")
    kq.kq_quantize_fp8_tensor(to_dev(bits), inv, y)
    ref = Qz.fp8_codes(W.bits_to_f32(bits), np.float32(inv))
    got = y.cpu().numpy()
    bad = np.nonzero(got != ref)
    assert bad[0].size == 0, (W.bits_to_f32(bits)[bad][:5], got[bad][:5], ref[bad][:5])


@pytest.mark.parametrize("cfg", [1, 2, 3])
def test_fp8_configs_bit_exact(cfg):
    print(f"fp8 cfg{cfg}", flush=True)
    qz = OP.quantize_inputs(*W.qkv_bits(cfg))
    c = W.config(cfg)
    for n, bits in zip("qkv", W.qkv_bits(cfg)):
        x = to_dev(bits)
        s, inv = kq.kq_fp8_scales_from_amax(_amax_gpu(x))
        assert (s, inv) == qz.scale[n]
        y = torch.empty_like(x, dtype=torch.uint8)
        kq.kq_quantize_fp8_tensor(x, inv, y)
        assert np.array_equal(y.cpu().numpy(), qz.codes[n])
        if n == "v":
            ld = kq.kq_vt_ld(c.N)
            yt = torch.empty((c.B * c.H, c.d, ld), dtype=torch.uint8, device="cuda")
            kq.kq_quantize_fp8_tensor(x, inv, yt, layout=kq.KQ_LAYOUT_TRANSPOSED)
            ref = np.zeros((c.B * c.H, c.d, ld), np.uint8)
            ref[:, :, :c.N] = qz.codes["v"].reshape(c.B * c.H, c.N, c.d).transpose(0, 2, 1)
            assert np.array_equal(yt.cpu().numpy(), ref)


@pytest.mark.parametrize("N", [1, 2, 63, 64, 65, 129, 255, 257, 1000])
def test_fp8_transposed_ragged(N):
    bits = W.random_bits(2, 3, N, 128, seed=100 + N, outliers=True)
    x = to_dev(bits)
    inv = np.float32(448.0) / np.float32(Qz.amax(W.bits_to_f32(bits)))
    ld = kq.kq_vt_ld(N)
    yt = torch.full((6, 128, ld), 0x55, dtype=torch.uint8, device="cuda")
    kq.kq_quantize_fp8_tensor(x, float(inv), yt, layout=kq.KQ_LAYOUT_TRANSPOSED)
    codes = Qz.fp8_codes(W.bits_to_f32(bits), inv).reshape(6, N, 128)
    ref = np.zeros((6, 128, ld), np.uint8)
    ref[:, :, :N] = codes.transpose(0, 2, 1)
    assert np.array_equal(yt.cpu().numpy(), ref)


# ---------------------------------------------------------------- FP4

def _fp4_gpu(x, rope=None, inv8=None):
    shape = tuple(x.shape)
    d = shape[-1]
    codes = torch.empty(shape[:-1] + (d // 2,), dtype=torch.uint8, device="cuda")
    scales = torch.empty(shape[:-1] + (d // 32,), dtype=torch.uint8, device="cuda")
    dq = torch.empty_like(x)
    fp8 = torch.empty(shape, dtype=torch.uint8, device="cuda") if inv8 is not None else None
    kq.kq_quantize_fp4_block(x, codes, scales, dq=dq, fp8=fp8,
                             inv_scale8=1.0 if inv8 is None else float(inv8), rope=rope)
    out = (codes.cpu().numpy(), scales.cpu().numpy(),
           dq.view(torch.int16).cpu().numpy().view(np.uint16))
    return out + ((fp8.cpu().numpy(),) if fp8 is not None else ())


def _check_fp4(got, x_f32, inv8=None):
    codes, scales, dq = Qz.fp4_block_quant(x_f32)
    assert np.array_equal(got[1], scales)
    bad = np.nonzero(got[0] != codes)
    assert bad[0].size == 0, (got[0][bad][:8], codes[bad][:8])
    assert np.array_equal(got[2], F.f32_to_bf16_bits_exact(dq))
    if inv8 is not None:
        assert np.array_equal(got[3], Qz.fp8_codes(dq, inv8))


@pytest.mark.parametrize("seed", [0, 1])
def test_fp4_every_bf16(seed):
    bits = all_finite_bf16_rows(seed=seed)
    inv8 = np.float32(0.37)
    _check_fp4(_fp4_gpu(to_dev(bits), inv8=inv8), W.bits_to_f32(bits), inv8)


def test_fp4_every_bf16_magnitude_within_blocks():
    # sorted magnitudes: every block holds neighbouring values, so all E8M0 exponents and
    # every position inside a block's range (ties, saturation, subnormals) are exercised
    bits = np.sort(all_finite_bf16_rows(seed=3).reshape(-1) & 0x7FFF).astype(np.uint16)
    bits = bits | (np.arange(bits.size, dtype=np.uint16) % 3 == 0).astype(np.uint16) << 15
    bits = bits.reshape(-1, 128)
    _check_fp4(_fp4_gpu(to_dev(bits), inv8=np.float32(5.5)), W.bits_to_f32(bits), np.float32(5.5))


def test_fp4_zero_and_tiny_blocks():
    x = np.zeros((4, 128), np.float32)
    x[1, 32:64] = np.float32(2.0 ** -130)
    x[1, 33] = -np.float32(2.0 ** -131)
    x[2, :] = -0.0
    x[3, 5] = np.float32(6.5e4)
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)
    _check_fp4(_fp4_gpu(to_dev(bits)), W.bits_to_f32(bits))


@pytest.mark.parametrize("cfg", [4, 5])
def test_fp4_configs_bit_exact(cfg):
    c = W.config(cfg)
    pos = W.positions(c) if c.rope else None
    table = None
    if c.rope:
        table = torch.from_numpy(kq.kq_rope3_table(pos)).cuda()
        otab = R.table(pos)
    for n, bits in zip("qkv", W.qkv_bits(cfg)):
        print(f"fp4 cfg{cfg} {n}", flush=True)
        x_f32 = W.bits_to_f32(bits)
        rope = None
        if c.rope and n in "qk":
            rope = (table, c.N)
            x_f32 = R.apply(x_f32, otab)
        inv8 = np.float32(448.0 / 5.0)
        _check_fp4(_fp4_gpu(to_dev(bits), rope=rope, inv8=inv8), x_f32, inv8)


def test_fp4_rope_ragged_tokens():
    pos = W.positions(W.config(5))[500:757]               # text/target boundary, 257 tokens
    table = torch.from_numpy(kq.kq_rope3_table(pos)).cuda()
    bits = W.random_bits(2, 2, len(pos), 128, seed=9, outliers=True)
    got = _fp4_gpu(to_dev(bits), rope=(table, len(pos)), inv8=np.float32(2.0))
    _check_fp4(got, R.apply(W.bits_to_f32(bits), R.table(pos)), np.float32(2.0))
