"""GPU parity of SVD-Quant in FP4 (kq_svdquant_down, kq_gemm_mxfp4_svdquant and its bf16 form)
against oracle/svdquant.py.

The oracle prepares the weights offline (float64 SVD of the planted-low-rank bf16 weights,
rank-r bf16 factors, bf16 residual); the device quantizes the residual and the activations
with its own FP4 encoder (codes must equal the oracle's bit for bit), forms T = bf16(A L_down^T)
and the fused GEMM C = dq(A4) dq(R4)^T + T L_up^T.  Bounds from the arithmetic:

  T: the device sums A L_down^T in float32 (error <= 2 K 2^-24 L1_T, L1_T = sum_k |a_k l_k|)
     before one rounding to bf16, so |T_gpu - T| <= 2^-7 |T| + 2 K 2^-24 L1_T (at most one bf16
     step where the float32 sum straddles a rounding point);
  C: the accumulators start from T L_up^T (r exact bf16 products) and add the MXFP4 products:
     |C_gpu - C| <= (K + r) 2^-24 L1_C + 2^-23 L1_C + sum_j |T_gpu - T|_j |L_up|_j, with
     L1_C = sum_k |dq a_k dq r_k| + sum_j |T_j L_up,j| (no truncation term: see
     test_gpu_gemm.py for the MXFP4 products).

Sizes: small ragged shapes (M, N tails inside a 256 x 256 tile, several k-steps, ranks 16, 32,
48) against the full oracle; the Kontext QKV projection (M = 8704, N = 9216, K = 3072) and the
output projection (N = 3072) at rank 32, compared on sampled rows over every column.
"""
import numpy as np
import pytest
import torch

import precision_quantized_attention_amd as kq
import workloads as W
from kq_testutil import to_dev
from oracle import quant as Qz
from oracle import svdquant as S

pytestmark = pytest.mark.gpu


def _bf16_dev(x):
    return to_dev(S.bf16_bits(x))


def _fp4_dev(x_dev):
    rows, K = x_dev.shape
    codes = torch.empty((rows, K // 2), dtype=torch.uint8, device="cuda")
    scales = torch.empty((rows, K // 32), dtype=torch.uint8, device="cuda")
    kq.kq_quantize_fp4_block(x_dev, codes, scales)
    return codes, scales


def _run(M, N, K, rank, seed, rows=None, out_bf16=False, fused=True):
    print(f"svdquant M={M} N={N} K={K} rank={rank} seed={seed}", flush=True)
    w = W.bits_to_f32(W.lowrank_weight_bits(N, K, seed))
    a_bits, _ = W.gemm_bits(M, 4, K, seed + 100)
    a = W.bits_to_f32(a_bits)
    l_up, l_down, r, rc_ref, rs_ref = S.quantize_weights(w, rank)
    # device: the residual's and the activations' FP4 codes, T, then the fused GEMM
    rc, rs = _fp4_dev(_bf16_dev(r))
    assert np.array_equal(rc.cpu().numpy(), rc_ref) and np.array_equal(rs.cpu().numpy(), rs_ref)
    a_dev = to_dev(a_bits)
    t = torch.empty((M, rank), dtype=torch.bfloat16, device="cuda")
    if fused:     # one pass over A: its MXFP4 codes and scales, and T
        ac = torch.empty((M, K // 2), dtype=torch.uint8, device="cuda")
        asc = torch.empty((M, K // 32), dtype=torch.uint8, device="cuda")
        kq.kq_svdquant_activations(a_dev, _bf16_dev(l_down), ac, asc, t)
    else:         # the block quantizer, then the down-projection alone
        ac, asc = _fp4_dev(a_dev)
        kq.kq_svdquant_down(a_dev, _bf16_dev(l_down), t)
    c = torch.empty((M, N), dtype=torch.bfloat16 if out_bf16 else torch.float32, device="cuda")
    fn = kq.kq_gemm_mxfp4_svdquant_bf16 if out_bf16 else kq.kq_gemm_mxfp4_svdquant
    fn(ac, asc, rc, rs, t, _bf16_dev(l_up), c)
    torch.cuda.synchronize()
    ac_all, as_all, _ = Qz.fp4_block_quant(a)
    assert np.array_equal(ac.cpu().numpy(), ac_all) and np.array_equal(asc.cpu().numpy(), as_all)
    rows = np.arange(M) if rows is None else np.asarray(rows)
    c_ref, t_ref = S.forward(a[rows], l_up, l_down, rc_ref, rs_ref)
    t_gpu = t.float().cpu().numpy()[rows].astype(np.float64)
    c_gpu = c.float().cpu().numpy()[rows].astype(np.float64)
    # bounds
    l1_t = np.abs(a[rows]).astype(np.float64) @ np.abs(l_down).T
    dt_bound = 2.0 ** -7 * np.abs(t_ref) + 2 * K * 2.0 ** -24 * l1_t
    dt = np.abs(t_gpu - t_ref)
    assert np.all(dt <= dt_bound), float(np.max(dt - dt_bound))
    ac_ref, as_ref, _ = Qz.fp4_block_quant(a[rows])
    l1_fp4 = np.abs(Qz.fp4_unpack(ac_ref, as_ref)) @ np.abs(Qz.fp4_unpack(rc_ref, rs_ref)).T
    l1_c = l1_fp4 + np.abs(t_ref) @ np.abs(l_up).T
    bound = (K + rank) * 2.0 ** -24 * l1_c + 2.0 ** -23 * l1_c + dt_bound @ np.abs(l_up).T
    if out_bf16:
        # one more rounding of the float32 result: half a bf16 step
        bound = bound + 2.0 ** -8 * (np.abs(c_ref) + bound)
    err = np.abs(c_gpu - c_ref)
    worst = np.unravel_index(np.argmax(err - bound), err.shape)
    print(f"  T equal {np.mean(dt == 0):.4f}, max |dC| / bound {np.max(err / np.maximum(bound, 1e-30)):.3f}, "
          f"branch share of |C| {np.linalg.norm(t_ref @ l_up.T) / np.linalg.norm(c_ref):.3f}", flush=True)
    assert np.all(err <= bound), (worst, err[worst], bound[worst])
    return c_gpu, c_ref


@pytest.mark.parametrize("M,N,K,rank", [(300, 260, 256, 16), (257, 512, 384, 32),
                                        (64, 132, 128, 48), (520, 300, 640, 64)])
def test_svdquant_small_shapes(M, N, K, rank):
    _run(M, N, K, rank, seed=M + N + K + rank)


def test_svdquant_down_projection_alone():
    """kq_svdquant_down after the block quantizer gives the same forward as the fused pass."""
    _run(300, 260, 256, 32, seed=77, fused=False)


def test_svdquant_bf16_output():
    _run(300, 260, 256, 32, seed=5, out_bf16=True)


def _rows(M, seed):
    rng = np.random.default_rng(seed)
    edges = [0, 1, 255, 256, 511, 512, M // 2, M - 257, M - 256, M - 2, M - 1]
    return np.unique(np.concatenate([edges, rng.choice(M, 53, replace=False)]))


@pytest.mark.parametrize("shape", W.GEMM_SHAPES, ids=lambda s: s.name)
def test_svdquant_kontext_shapes(shape):
    _run(shape.M, shape.N, shape.K, 32, seed=21, rows=_rows(shape.M, 3))


def test_svdquant_branch_lowers_the_error():
    """Against the exact bf16 GEMM, the device's SVD-Quant output at rank 32 is several times
    closer than its plain MXFP4 GEMM of the same weights (the planted outliers go to the
    branch)."""
    M, N, K = 512, 384, 512
    w_bits = W.lowrank_weight_bits(N, K, 9)
    a_bits, _ = W.gemm_bits(M, 4, K, 9 + 100)          # the activations _run draws
    exact = W.bits_to_f32(a_bits).astype(np.float64) @ W.bits_to_f32(w_bits).astype(np.float64).T
    c_sq, _ = _run(M, N, K, 32, seed=9)
    ac, asc = _fp4_dev(to_dev(a_bits))
    wc, wsc = _fp4_dev(to_dev(w_bits))
    c0 = torch.empty((M, N), dtype=torch.float32, device="cuda")
    kq.kq_gemm_mxfp4(ac, asc, wc, wsc, c0)
    c0 = c0.cpu().numpy().astype(np.float64)
    e_sq = np.linalg.norm(c_sq - exact) / np.linalg.norm(exact)
    e_0 = np.linalg.norm(c0 - exact) / np.linalg.norm(exact)
    print(f"  rel-L2 vs exact bf16 GEMM: plain MXFP4 {e_0:.4f}, SVD-Quant r=32 {e_sq:.4f}", flush=True)
    assert e_sq < e_0 / 2
