"""Host-side checks of the C ABI (no GPU needed): the library loads, exports every entry point
include/kq.h declares, validates arguments before touching HIP, and its two host-only
helpers (scale rule, rotary table) agree bit-exactly with the oracle's own versions."""
import ctypes
import os
import re

import numpy as np
import pytest

import precision_quantized_attention_amd as kq
import workloads as W
from oracle import quant as Qz
from oracle import rope as R

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.skipif(not os.path.exists(kq.LIB_PATH),
                                reason="libkq.so not built (run __graft_entry__.build())")


def _declared():
    src = open(os.path.join(ROOT, "include", "kq.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kq_[a-z0-9_]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    names = _declared()
    assert set(names) >= {"kq_amax_calibrate", "kq_quantize_fp8_tensor", "kq_quantize_fp4_block",
                          "kq_attn_quant_fwd", "kq_fp8_scales_from_amax", "kq_rope3_table",
                          "kq_vt_ld", "kq_status_string"}
    lib = ctypes.CDLL(kq.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings_and_vt_ld():
    assert kq.kq_status_string(0) == "ok"
    assert "invalid" in kq.kq_status_string(-1)
    assert kq.kq_vt_ld(1) == 128 and kq.kq_vt_ld(128) == 128 and kq.kq_vt_ld(129) == 256
    assert kq.kq_vt_ld(8704) == 8704 and kq.kq_vt_ld(0) == -1


def test_validation_rejects_before_any_hip_call():
    lib = kq.load()
    INVALID, UNSUPPORTED = -1, -2
    fake = ctypes.c_void_p(0x10000)          # aligned, never dereferenced: rejected earlier
    odd = ctypes.c_void_p(0x10008)
    assert lib.kq_amax_calibrate(None, 10, fake, None) == INVALID
    assert lib.kq_amax_calibrate(fake, -1, fake, None) == INVALID
    assert lib.kq_amax_calibrate(odd, 10, fake, None) == INVALID
    assert lib.kq_amax_calibrate(fake, 0, fake, None) == 0          # n == 0: nothing enqueued
    assert lib.kq_quantize_fp8_tensor(None, 4, 128, 0, 1.0, fake, 0, None) == INVALID
    assert lib.kq_quantize_fp8_tensor(fake, 4, 128, 0, float("nan"), fake, 0, None) == INVALID
    assert lib.kq_quantize_fp8_tensor(fake, 4, 128, 0, -1.0, fake, 0, None) == INVALID
    assert lib.kq_quantize_fp8_tensor(fake, 4, 120, 0, 1.0, fake, 0, None) == UNSUPPORTED
    assert lib.kq_quantize_fp8_tensor(fake, 4, 128, 3, 1.0, fake, 1, None) == INVALID
    assert lib.kq_quantize_fp8_tensor(fake, 4, 64, 4, 1.0, fake, 1, None) == UNSUPPORTED
    assert lib.kq_quantize_fp8_tensor(fake, 4, 128, 4, 1.0, fake, 7, None) == INVALID
    assert lib.kq_quantize_fp4_block(fake, 4, 48, fake, fake, None, None, 1.0, None,
                                     None) == UNSUPPORTED
    assert lib.kq_quantize_fp4_block(fake, 4, 128, None, fake, None, None, 1.0, None,
                                     None) == INVALID
    assert lib.kq_quantize_fp4_block(fake, 4, 128, fake, fake, None, fake, 0.0, None,
                                     None) == INVALID
    A = lib.kq_attn_quant_fwd
    assert A(fake, fake, fake, 1, 1, 1, 128, 128, 1.0, 1.0, 1.0, 0.1, None, None, None) == INVALID
    assert A(fake, fake, fake, 1, 1, 1, 128, 64, 1.0, 1.0, 1.0, 0.1, fake, None, None) == UNSUPPORTED
    assert A(fake, fake, fake, 0, 1, 1, 128, 128, 1.0, 1.0, 1.0, 0.1, fake, None, None) == UNSUPPORTED
    assert A(fake, fake, fake, 1, 0, 1, 128, 128, 1.0, 1.0, 1.0, 0.1, fake, None, None) == INVALID
    assert A(fake, fake, fake, 1, 1, 1, 0, 128, 1.0, 1.0, 1.0, 0.1, fake, None, None) == INVALID
    assert A(fake, fake, fake, 1, 1, 1, 128, 128, 0.0, 1.0, 1.0, 0.1, fake, None, None) == INVALID
    assert A(fake, fake, fake, 1, 1, 1, 128, 128, 1.0, float("inf"), 1.0, 0.1, fake, None,
             None) == INVALID
    assert A(odd, fake, fake, 1, 1, 1, 128, 128, 1.0, 1.0, 1.0, 0.1, fake, None, None) == INVALID
    assert A(fake, fake, fake, 5, 1, 1, 128, 128, 1.0, 1.0, 1.0, 0.1, fake, None, None) == INVALID
    W = lib.kq_attn_quant_fwd_ws                 # same checks, then the workspace alignment
    assert W(fake, fake, fake, 1, 1, 1, 128, 128, 1.0, 1.0, 1.0, 0.1, None, None, fake, 1 << 20,
             None) == INVALID
    assert W(fake, fake, fake, 1, 1, 1, 128, 64, 1.0, 1.0, 1.0, 0.1, fake, None, fake, 1 << 20,
             None) == UNSUPPORTED
    assert W(fake, fake, fake, 1, 1, 1, 128, 128, 1.0, 1.0, 1.0, 0.1, fake, None, odd, 1 << 20,
             None) == INVALID
    Fq = lib.kq_attn_quant_fwd_qbf16             # Q's scale, the attention checks, the workspace
    assert Fq(fake, 0.0, fake, fake, 1, 1, 1, 128, 128, 1.0, 1.0, 1.0, 0.1, fake, None, None, 0,
              None) == INVALID
    assert Fq(fake, float("inf"), fake, fake, 1, 1, 1, 128, 128, 1.0, 1.0, 1.0, 0.1, fake, None,
              None, 0, None) == INVALID
    assert Fq(None, 2.0, fake, fake, 1, 1, 1, 128, 128, 1.0, 1.0, 1.0, 0.1, fake, None, None, 0,
              None) == INVALID
    assert Fq(odd, 2.0, fake, fake, 1, 1, 1, 128, 128, 1.0, 1.0, 1.0, 0.1, fake, None, None, 0,
              None) == INVALID
    assert Fq(fake, 2.0, fake, fake, 1, 1, 1, 128, 64, 1.0, 1.0, 1.0, 0.1, fake, None, None, 0,
              None) == UNSUPPORTED
    assert Fq(fake, 2.0, fake, fake, 1, 1, 1, 128, 128, 1.0, 1.0, 1.0, 0.1, fake, None, odd,
              1 << 20, None) == INVALID
    Z = lib.kq_attn_quant_fwd_noalloc            # the attention checks, before any HIP call
    assert Z(fake, fake, fake, 1, 1, 1, 128, 128, 1.0, 1.0, 1.0, 0.1, None, None, None) == INVALID
    assert Z(fake, fake, fake, 1, 1, 1, 128, 64, 1.0, 1.0, 1.0, 0.1, fake, None, None) == UNSUPPORTED
    assert Z(fake, fake, fake, 1, 1, 1, 128, 128, 1.0, 1.0, float("nan"), 0.1, fake, None,
             None) == INVALID
    assert Z(odd, fake, fake, 1, 1, 1, 128, 128, 1.0, 1.0, 1.0, 0.1, fake, None, None) == INVALID
    n = ctypes.c_size_t(0)
    S = lib.kq_attn_workspace_size
    assert S(1, 1, 128, 128, None) == INVALID
    assert S(0, 1, 128, 128, ctypes.byref(n)) == INVALID
    assert S(1, 1, 0, 128, ctypes.byref(n)) == INVALID
    assert S(1, 1, 128, 64, ctypes.byref(n)) == UNSUPPORTED
    X = lib.kq_attn_mxfp4_fwd                   # the attention checks, then the scales
    assert X(fake, None, fake, fake, fake, 1, 1, 1, 128, 128, 1.0, 0.1, fake, None, None, 0,
             None) == INVALID
    assert X(fake, fake, fake, ctypes.c_void_p(0x10002), fake, 1, 1, 1, 128, 128, 1.0, 0.1, fake,
             None, None, 0, None) == INVALID
    assert X(fake, fake, fake, fake, fake, 1, 1, 1, 128, 64, 1.0, 0.1, fake, None, None, 0,
             None) == UNSUPPORTED
    assert X(fake, fake, fake, fake, fake, 1, 1, 1, 128, 128, 0.0, 0.1, fake, None, None, 0,
             None) == INVALID
    assert X(fake, fake, None, fake, fake, 1, 1, 1, 128, 128, 1.0, 0.1, fake, None, None, 0,
             None) == INVALID
    assert X(fake, fake, fake, fake, fake, 1, 1, 1, 128, 128, 1.0, 0.1, fake, None, odd, 1 << 20,
             None) == INVALID
    R1, RS, RA = lib.kq_attn_r1_fwd, lib.kq_attn_r1_stats, lib.kq_attn_r1_amax
    assert R1(fake, fake, fake, 1, 1, 1, 128, 128, 1.0, 1.0, 1.0, 0.1, 0.0, fake, fake,
              None, 0, None) == INVALID                                         # amax_P 0
    assert R1(fake, fake, fake, 1, 1, 1, 128, 128, 1.0, 1.0, 1.0, 0.1, float("inf"), fake,
              fake, None, 0, None) == INVALID
    assert R1(fake, fake, fake, 1, 1, 1, 128, 128, 1.0, 1.0, 1.0, 0.1, 0.5, fake, None,
              None, 0, None) == INVALID                                         # no stats
    assert R1(fake, fake, fake, 1, 1, 1, 128, 128, 1.0, 1.0, 1.0, 0.1, 0.5, fake, odd,
              None, 0, None) == INVALID
    assert R1(fake, fake, fake, 1, 1, 1, 128, 64, 1.0, 1.0, 1.0, 0.1, 0.5, fake, fake,
              None, 0, None) == UNSUPPORTED
    assert R1(fake, fake, fake, 1, 1, 1, 128, 128, 1.0, 1.0, 1.0, 0.1, 0.5, fake, fake,
              odd, 1 << 20, None) == INVALID                                    # workspace
    assert RS(fake, fake, fake, 1, 1, 1, 128, 128, 1.0, 1.0, 1.0, 0.1, None, None, 0,
              None) == INVALID
    assert RS(fake, fake, fake, 1, 0, 1, 128, 128, 1.0, 1.0, 1.0, 0.1, fake, None, 0,
              None) == INVALID
    assert RS(fake, fake, fake, 1, 1, 1, 128, 128, 1.0, 1.0, 1.0, 0.1, odd, None, 0,
              None) == INVALID
    assert RA(None, 4, fake, None) == INVALID
    assert RA(fake, 0, fake, None) == INVALID
    assert RA(odd, 4, fake, None) == INVALID
    G8, G4 = lib.kq_gemm_fp8, lib.kq_gemm_mxfp4
    assert G8(fake, fake, 256, 256, 256, 1.0, 1.0, None, None) == INVALID
    assert G8(None, fake, 256, 256, 256, 1.0, 1.0, fake, None) == INVALID
    assert G8(odd, fake, 256, 256, 256, 1.0, 1.0, fake, None) == INVALID
    assert G8(fake, fake, 0, 256, 256, 1.0, 1.0, fake, None) == INVALID
    assert G8(fake, fake, 256, 256, -64, 1.0, 1.0, fake, None) == INVALID
    assert G8(fake, fake, 256, 256, 256, 0.0, 1.0, fake, None) == INVALID
    assert G8(fake, fake, 256, 256, 256, 1.0, float("nan"), fake, None) == INVALID
    assert G8(fake, fake, 256, 256, 256, 3e38, 3e38, fake, None) == INVALID    # s_a s_b = inf
    assert G8(fake, fake, 256, 256, 96, 1.0, 1.0, fake, None) == UNSUPPORTED   # K % 64
    assert G8(fake, fake, 256, 258, 256, 1.0, 1.0, fake, None) == UNSUPPORTED  # N % 4
    assert G8(fake, fake, 1 << 20, 256, 4096, 1.0, 1.0, fake, None) == UNSUPPORTED  # > 2^31 B
    assert G4(fake, fake, fake, fake, 256, 256, 256, None, None) == INVALID
    assert G4(fake, None, fake, fake, 256, 256, 256, fake, None) == INVALID
    assert G4(fake, fake, fake, ctypes.c_void_p(0x10002), 256, 256, 256, fake, None) == INVALID
    assert G4(fake, fake, fake, fake, 256, 256, 192, fake, None) == UNSUPPORTED  # K % 128
    assert G4(fake, fake, fake, fake, 256, 6, 256, fake, None) == UNSUPPORTED    # N % 4
    # the bf16-output forms share the validation
    B8, B4 = lib.kq_gemm_fp8_bf16, lib.kq_gemm_mxfp4_bf16
    assert B8(fake, fake, 256, 256, 256, 1.0, 1.0, None, None) == INVALID
    assert B8(fake, fake, 256, 256, 256, 1.0, 1.0, odd, None) == INVALID
    assert B8(fake, fake, 256, 256, 256, -1.0, 1.0, fake, None) == INVALID
    assert B8(fake, fake, 256, 256, 96, 1.0, 1.0, fake, None) == UNSUPPORTED   # K % 64
    assert B8(fake, fake, 256, 258, 256, 1.0, 1.0, fake, None) == UNSUPPORTED  # N % 4
    assert B4(fake, None, fake, fake, 256, 256, 256, fake, None) == INVALID
    assert B4(fake, fake, fake, fake, 256, 256, 192, fake, None) == UNSUPPORTED  # K % 128


def test_scale_rule_matches_oracle():
    rng = np.random.default_rng(0)
    amaxes = np.concatenate([[0.0, 448.0, 1.0, 3.5, 1e-30, 3e38],
                             np.exp(rng.uniform(-20, 20, 2000))]).astype(np.float32)
    for a in amaxes:
        s, inv = kq.kq_fp8_scales_from_amax(float(a))
        so, invo = Qz.fp8_scales(float(a))
        assert s == so and inv == invo, a
    with pytest.raises(kq.KQError):
        kq.kq_fp8_scales_from_amax(-1.0)


def test_rope_table_matches_oracle_bit_exactly():
    for cfg in (5, 3):
        pos = W.positions(W.config(cfg))
        ours = kq.kq_rope3_table(pos)
        ref = R.table(pos)
        assert ours.dtype == np.float32 and ours.shape == ref.shape
        assert np.array_equal(ours.view(np.uint32), ref.view(np.uint32))
