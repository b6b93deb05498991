"""Pins for the oracle's number formats (E4M3, E2M1, E8M0).

Each pin is independent of the code it checks: OCP specification values
(tests/golden), torch's own float8_e4m3fn conversion on the CPU, and brute-force
searches written here from scratch.
"""
import math
import os

import numpy as np
import pytest
import torch

from oracle import formats as F
from oracle import quant as Qz

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_table(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                rows.append(line.split())
    return rows


def _all_finite_bf16():
    bits = np.arange(1 << 16, dtype=np.uint32)
    exp = (bits >> 7) & 0xFF
    bits = bits[exp != 0xFF]
    return (bits << 16).view(np.float32)


def _same(a, b):
    a = float(a)
    b = float(b)
    if math.isnan(b):
        return math.isnan(a)
    return a == b and math.copysign(1, a) == math.copysign(1, b)


# ---------------------------------------------------------------- E4M3

def test_e4m3_spec_points():
    for code, value in _read_table("e4m3_ocp_fp8.txt"):
        assert _same(F.e4m3_decode(int(code, 16)), float(value)), code


def test_e4m3_decode_matches_torch_for_all_codes():
    t = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = F.e4m3_decode(np.arange(256))
    for c in range(256):
        assert _same(ours[c], t[c]), hex(c)


def test_e4m3_encode_matches_torch_on_every_bf16_and_scales():
    x = _all_finite_bf16()
    for scale in (1.0, 3.7, 0.013, 448.0 / 3.0, 1e-3, 2.0 ** -7):
        with np.errstate(over="ignore"):
            y = (x * np.float32(scale)).astype(np.float32)
        y = y[np.abs(y) < 1e30]
        ours = F.e4m3_encode(y)
        ref = torch.from_numpy(np.clip(y, -448, 448)).to(torch.float8_e4m3fn).view(
            torch.uint8).numpy()
        bad = np.nonzero(ours != ref)[0]
        assert bad.size == 0, (scale, y[bad[:5]], ours[bad[:5]], ref[bad[:5]])


def test_e4m3_encode_midpoints_go_to_even_code():
    mags = F.e4m3_decode(np.arange(0x7F))
    for c in range(0x7E):
        mid = (mags[c] + mags[c + 1]) / 2.0           # exact in float64
        want = c if c % 2 == 0 else c + 1
        assert F.e4m3_encode(mid) == want, (c, mid)
        assert F.e4m3_encode(-mid) == (want | 0x80)
        assert F.e4m3_encode(np.nextafter(mid, 0.0)) == c
        assert F.e4m3_encode(np.nextafter(mid, 1e9)) == c + 1


def test_e4m3_saturates_and_keeps_sign_of_zero():
    assert F.e4m3_encode(464.0) == 0x7E
    assert F.e4m3_encode(1e6) == 0x7E
    assert F.e4m3_encode(-1e6) == 0xFE
    assert F.e4m3_encode(-0.0) == 0x80
    assert F.e4m3_encode(-1e-9) == 0x80
    assert F.e4m3_encode(2.0 ** -10) == 0x00            # tie between 0 and 2^-9 -> even code
    assert F.e4m3_encode(3.0 * 2.0 ** -10) == 0x02      # tie between codes 1 and 2


def test_e4m3_encode_matches_brute_force_random():
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.standard_normal(20000) * s for s in (1e-3, 0.1, 1, 30, 300)])
    x = x.astype(np.float32).astype(np.float64)
    mags = F.e4m3_decode(np.arange(0x7F))
    ours = F.e4m3_encode(x)
    for xi, ci in zip(x[:3000], ours[:3000]):
        a = min(abs(xi), 448.0)
        dist = np.abs(mags - a)
        best = np.nonzero(dist == dist.min())[0]
        want = best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0]
        want |= 0x80 if math.copysign(1, xi) < 0 else 0
        assert ci == want, (xi, ci, want)


# ---------------------------------------------------------------- E2M1

def test_e2m1_spec_values():
    for code, value in _read_table("e2m1_ocp_mx.txt"):
        assert _same(F.e2m1_decode(int(code, 16)), float(value)), code


def test_e2m1_rounding_table():
    for x, code in _read_table("e2m1_rounding.txt"):
        xv = float(np.float32(float(x)))
        assert int(F.e2m1_encode(xv)) == int(code, 16), x


def test_e2m1_encode_matches_brute_force():
    vals = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.uniform(-8, 8, 4000), np.arange(-70, 71) / 10.0,
                        np.arange(-28, 29) / 4.0])
    ours = F.e2m1_encode(x)
    for xi, ci in zip(x, ours):
        a = min(abs(xi), 6.0)
        d = [abs(a - v) for v in vals]
        m = min(d)
        cands = [i for i, di in enumerate(d) if di == m]
        want = cands[0] if len(cands) == 1 else [c for c in cands if c % 2 == 0][0]
        if math.copysign(1, xi) < 0:
            want |= 8
        assert ci == want, (xi, ci, want)


# ---------------------------------------------------------------- E8M0 exponent rule

def test_e8m0_exponent_is_floor_log2_minus_2_on_every_bf16():
    x = _all_finite_bf16()
    x = np.unique(np.abs(x[~np.isnan(x)])).astype(np.float64)
    for a in x[::7]:
        if a == 0:
            want = -127
        else:
            E = 0
            while 2.0 ** E > a:
                E -= 1
            while 2.0 ** (E + 1) <= a:
                E += 1
            want = max(-127, min(127, E - 2))
        assert Qz.e8m0_exponent(a) == want, a


def test_e8m0_decode():
    assert F.e8m0_decode(127) == 1.0
    assert F.e8m0_decode(0) == 2.0 ** -127
    assert F.e8m0_decode(254) == 2.0 ** 127
    assert np.isnan(F.e8m0_decode(255))
