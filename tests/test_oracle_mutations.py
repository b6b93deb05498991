"""Plant plausible mistakes in the oracle (on the CPU, via monkeypatch) and check that the
pins catch each one.  This shows the pins are sensitive to the errors they guard against."""
import numpy as np
import pytest

import test_oracle_attention as TA
import test_oracle_formats as TF
import test_oracle_gemm as TG
import test_oracle_quant as TQ
from oracle import attention as A
from oracle import formats as F
from oracle import gemm as G
from oracle import quant as Qz
from oracle import rope as R


def _caught(pins):
    for pin in pins:
        try:
            pin()
        except Exception:
            return True
    return False


def _ties_down(a, mags):
    hi = np.clip(np.searchsorted(mags, a, side="left"), 1, len(mags) - 1)
    lo = hi - 1
    idx = np.where(mags[hi] - a < a - mags[lo], hi, lo)
    idx = np.where(a <= mags[0], 0, idx)
    return np.where(a >= mags[-1], len(mags) - 1, idx)


def _r3_floor(Qv, Kv, Vv, c1, c2, quantize_p=True):
    raw = Qv @ Kv.T
    t = F.fl32(raw * float(c1)).astype(np.float64)
    M = np.floor(np.max(t, axis=1, keepdims=True))             # planted: floor, not ceil
    p = F.fl32(np.exp2(t - M))
    l = F.fl32(np.sum(p.astype(np.float64), axis=1))
    pv = F.e4m3_decode(F.e4m3_encode(p * np.float32(448))) if quantize_p else p * 448.0
    return F.fl32(pv @ Vv * float(c2) / l.astype(np.float64)[:, None]), M[:, 0], l


def _r3_sum_of_quantized(Qv, Kv, Vv, c1, c2, quantize_p=True):
    raw = Qv @ Kv.T
    t = F.fl32(raw * float(c1)).astype(np.float64)
    M = np.ceil(np.max(t, axis=1, keepdims=True))
    p = F.fl32(np.exp2(t - M))
    pv = F.e4m3_decode(F.e4m3_encode(p * np.float32(448))) if quantize_p else p * 448.0
    l = F.fl32(np.sum(pv, axis=1) / 448.0)                     # planted: sum of quantized P
    return F.fl32(pv @ Vv * float(c2) / l.astype(np.float64)[:, None]), M[:, 0], l


def _apply_wrong_sign(x_f32, tab):
    x = np.asarray(x_f32, dtype=np.float32)
    c, s = tab[:, :, 0], tab[:, :, 1]
    y = np.empty_like(x)
    y[..., 0::2] = x[..., 0::2] * c + x[..., 1::2] * s          # planted: clockwise rotation
    y[..., 1::2] = x[..., 1::2] * c - x[..., 0::2] * s
    return y


def _gemm_fp8_no_weight_scale(a8, b8, s_a, s_b):
    return (F.e4m3_decode(a8) @ F.e4m3_decode(b8).T) * float(s_a)     # planted: s_b dropped


def _unpack_high_nibble_first(codes, scales, block=32):
    codes = np.asarray(codes, dtype=np.uint8)
    c = np.stack([codes >> 4, codes & 0xF], axis=-1).reshape(codes.shape[:-1] + (-1,))
    return F.e2m1_decode(c) * F.e8m0_decode(np.repeat(np.asarray(scales), block, axis=-1))


def _unpack_block_16(codes, scales, block=32):
    codes = np.asarray(codes, dtype=np.uint8)
    c = np.stack([codes & 0xF, codes >> 4], axis=-1).reshape(codes.shape[:-1] + (-1,))
    s = np.repeat(np.asarray(scales), 16, axis=-1)                   # planted: 16-blocks
    s = np.concatenate([s, s], axis=-1)[..., : c.shape[-1]]
    return F.e2m1_decode(c) * F.e8m0_decode(s)


def _unpack_ignoring_scales(codes, scales, block=32):
    codes = np.asarray(codes, dtype=np.uint8)
    c = np.stack([codes & 0xF, codes >> 4], axis=-1).reshape(codes.shape[:-1] + (-1,))
    return F.e2m1_decode(c)                                          # planted: no 2^e


def _r1_variant(normalize_p: bool, amax_of_normalized: bool):
    def r1(q8, k8, v8, s_q, s_k, s_v, sm_scale, amax_p=None, rows=None):
        B, H, N, d = q8.shape
        rows = np.arange(N) if rows is None else np.asarray(rows)
        c1, _ = A.constants(s_q, s_k, s_v, sm_scale)
        Ps, ps = [], []
        for b in range(B):
            for h in range(H):
                raw = F.e4m3_decode(q8[b, h, rows]) @ F.e4m3_decode(k8[b, h]).T
                t = F.fl32(raw * float(c1)).astype(np.float64)
                p = F.fl32(np.exp2(t - np.ceil(np.max(t, axis=1, keepdims=True))))
                l = F.fl32(np.sum(p.astype(np.float64), axis=1))
                ps.append(p)
                Ps.append(p / l[:, None] if normalize_p else p)
        if amax_p is None:
            amax_p = max(float(np.max(P)) for P in (Ps if amax_of_normalized else ps))
        s_p = np.float32(np.float32(amax_p) / np.float32(448))
        inv_p = np.float32(np.float32(448) / np.float32(amax_p))
        O = np.empty((B, H, len(rows), d), np.float32)
        for i, P in enumerate(Ps):
            b, h = divmod(i, H)
            pq = F.e4m3_decode(F.e4m3_encode(P * inv_p)) * float(s_p)
            O[b, h] = F.fl32(pq @ (F.e4m3_decode(v8[b, h]) * float(np.float32(s_v))))
        return O, amax_p
    return r1


MUTATIONS = {
    "r1 without the 1/l normalization": (
        lambda mp: mp.setattr(A, "attention_r1", _r1_variant(False, False)),
        [TA._pin_r1_closed_form]),
    "r1 amax_P calibrated on the unnormalized p": (
        lambda mp: mp.setattr(A, "attention_r1", _r1_variant(True, False)),
        [TA._pin_r1_closed_form]),
    "mxfp4 attention with 16-element scale blocks": (
        lambda mp: mp.setattr(Qz, "fp4_unpack", _unpack_block_16),
        [TA._pin_r3_mxfp4_equals_fp8_r3]),
    "mxfp4 attention ignores block scales": (
        lambda mp: mp.setattr(Qz, "fp4_unpack", _unpack_ignoring_scales),
        [TA._pin_r3_mxfp4_equals_fp8_r3]),
    "gemm fp8 weight scale dropped": (lambda mp: mp.setattr(G, "gemm_fp8", _gemm_fp8_no_weight_scale),
                                      [TG.test_fp8_all_ones_closed_form,
                                       TG.test_fp8_one_hot_rows_select_weight_columns]),
    "fp4 unpack high nibble first": (lambda mp: mp.setattr(Qz, "fp4_unpack", _unpack_high_nibble_first),
                                     [TG.test_mxfp4_one_hot_rows_select_weight_columns]),
    "fp4 unpack 16-element blocks": (lambda mp: mp.setattr(Qz, "fp4_unpack", _unpack_block_16),
                                     [TG.test_mxfp4_hand_computed_example]),
    "e4m3/e2m1 ties round down": (lambda mp: mp.setattr(F, "_nearest_code", _ties_down),
                                  [TF.test_e4m3_encode_midpoints_go_to_even_code,
                                   TF.test_e2m1_rounding_table]),
    "fp4 exponent off by one": (lambda mp: mp.setattr(
        Qz, "e8m0_exponent",
        lambda a: -127 if a == 0 else max(-127, min(127, int(np.floor(np.log2(a))) - 1))),
        [TQ.test_fp4_worked_block]),
    "fp8 scale inverted": (lambda mp: mp.setattr(
        Qz, "fp8_scales", lambda a: (np.float32(448.0 / a) if a else np.float32(1),
                                     np.float32(a / 448.0) if a else np.float32(1))),
        [TQ.test_fp8_scale_rule, TQ.test_fp8_amax_maps_to_max_code]),
    "row offset uses floor": (lambda mp: mp.setattr(A, "r3_rows", _r3_floor),
                              [TA._pin_softmax_invariants, TA._pin_r3_against_torch_fp8_cast]),
    "P scale 256 instead of 448": (lambda mp: mp.setattr(A, "P_SCALE", 256.0),
                                   [TA._pin_r3_against_torch_fp8_cast]),
    "row sum of quantized P": (lambda mp: mp.setattr(A, "r3_rows", _r3_sum_of_quantized),
                               [TA._pin_r3_against_torch_fp8_cast]),
    "softmax scale dropped": (lambda mp: mp.setattr(
        A, "constants", lambda s_q, s_k, s_v, sm: (np.float32(float(s_q) * float(s_k) * A.LOG2E),
                                                   np.float32(float(s_v) / 448.0))),
        [TA._pin_unquantized_equals_sdpa]),
    "rope rotates clockwise": (lambda mp: mp.setattr(R, "apply", _apply_wrong_sign),
                               [TQ.test_rope_rotates_counterclockwise_and_text_unchanged]),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    plant, pins = MUTATIONS[name]
    assert not _caught(pins), "pins must pass on the unmodified oracle"
    plant(monkeypatch)
    assert _caught(pins), f"no pin caught: {name}"
