"""The library's offline SVD-Quant weight step (kq_svdquant_factorize, host code, no GPU)
against the oracle's float64 SVD (oracle/svdquant.py).

Where singular value r stands clear of the rest (the planted rank of the synthetic weights)
the leading subspace is well defined and both sides must give the same bf16 factor product and
the same bf16 residual bit for bit.  Past the planted rank the remaining singular values are a
flat noise spectrum whose directions no two SVD routes need agree on; there the residual's
energy must stay within 1% of the Eckart-Young optimum the oracle's exact SVD attains."""
import numpy as np
import pytest

import precision_quantized_attention_amd as kq
import workloads as W
from oracle import svdquant as S


def _f(bits):
    return W.bits_to_f32(bits).astype(np.float64)


@pytest.mark.parametrize("N,K", [(256, 128), (384, 512), (1024, 256)])
def test_factorization_matches_the_oracle_at_the_planted_rank(N, K):
    wb = W.lowrank_weight_bits(N, K, 31)
    lu, ld, rb = kq.kq_svdquant_factorize(wb, W.PLANTED_RANK)
    lu_o, ld_o, r_o, _, _ = S.quantize_weights(_f(wb).astype(np.float32), W.PLANTED_RANK)
    assert np.array_equal(_f(lu) @ _f(ld), lu_o @ ld_o)
    assert np.array_equal(_f(rb), r_o)


@pytest.mark.parametrize("N,K,rank", [(256, 128, 16), (512, 384, 32)])
def test_residual_energy_past_the_planted_rank(N, K, rank):
    wb = W.lowrank_weight_bits(N, K, 33)
    lu, ld, rb = kq.kq_svdquant_factorize(wb, rank)
    _, _, r_o, _, _ = S.quantize_weights(_f(wb).astype(np.float32), rank)
    ratio = np.linalg.norm(_f(rb)) / np.linalg.norm(r_o)
    assert 0.999 <= ratio <= 1.01, ratio
    gram = _f(ld) @ _f(ld).T                 # L_down's rows: orthonormal up to bf16 rounding
    assert np.max(np.abs(gram - np.eye(rank))) < 2 ** -6


def test_factorize_rejects_bad_arguments():
    wb = W.lowrank_weight_bits(64, 32, 1)
    for r in (0, 33):
        with pytest.raises(kq.KQError):
            kq.kq_svdquant_factorize(wb, r)
    bad = wb.copy()
    bad[3, 4] = 0x7FC0                       # NaN
    with pytest.raises(kq.KQError):
        kq.kq_svdquant_factorize(bad, 4)
