"""Pins of the SVD-Quant oracle (oracle/svdquant.py), each independent of the code it checks:
torch's bf16 cast, the MXFP4 GEMM oracle at rank 0, a hand-worked rank-1 case, the
Eckart-Young bound on the residual, and orthonormal factors.  Planted mistakes at the end
show the pins catch them."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import gemm as G
from oracle import quant as Q
from oracle import svdquant as S


def test_bf16_round_matches_torch_cast_and_ties_go_to_even():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(200000) * 10 ** rng.uniform(-6, 6, 200000),
                        [1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 3.0, 0.0]]).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy().astype(np.float64)
    assert np.array_equal(S.bf16_round(x), want)
    assert S.bf16_round(np.array([1 + 2 ** -8]))[0] == 1.0              # tie: even mantissa
    assert S.bf16_round(np.array([1 + 3 * 2 ** -8]))[0] == 1 + 2 ** -6


def _acts(M, K, seed):
    a_bits, _ = W.gemm_bits(M, 32, K, seed)
    return W.bits_to_f32(a_bits)


def test_rank_zero_is_the_mxfp4_gemm_of_the_weights():
    """Without the branch the residual is W itself (already bf16), so the forward is the MXFP4
    GEMM oracle of FP4(A) and FP4(W), bit for bit."""
    w = W.bits_to_f32(W.lowrank_weight_bits(96, 128, 3))
    a = _acts(40, 128, 4)
    l_up, l_down, r, rc, rs = S.quantize_weights(w, 0)
    assert np.array_equal(r, w.astype(np.float64))
    c, t = S.forward(a, l_up, l_down, rc, rs)
    ac, asc, _ = Q.fp4_block_quant(a)
    wc, wsc, _ = Q.fp4_block_quant(w)
    assert t.shape == (40, 0)
    assert np.array_equal(c, G.gemm_mxfp4(ac, asc, wc, wsc).astype(np.float32))


def test_hand_worked_rank_one_case():
    """W = (3, 4)^T (1/4 on 16 of 32 columns): singular value 5, u = (0.6, 0.8), v = 1/4 on
    those columns.  Rank 1 takes all of W (L_up = +-(3, 4), L_down = +-v), the residual is 0,
    and for A rows of 16 ones and 16 halves (then zeros) T = 4 and 2 (same sign as L_down), so
    C = T L_up^T = (12, 16) and (6, 8)."""
    v = np.zeros(32)
    v[:16] = 0.25
    w = np.outer([3.0, 4.0], v).astype(np.float32)
    l_up, l_down, r, rc, rs = S.quantize_weights(w, 1)
    sgn = np.sign(l_up[0, 0])
    assert np.array_equal(l_up[:, 0], sgn * np.array([3.0, 4.0]))
    assert np.array_equal(l_down[0], sgn * v)
    assert not np.any(r) and not np.any(rc & 0x7)                       # zero residual codes
    a = np.zeros((2, 32), np.float32)
    a[0, :16], a[1, :16] = 1.0, 0.5
    c, t = S.forward(a, l_up, l_down, rc, rs)
    assert np.array_equal(t[:, 0], sgn * np.array([4.0, 2.0]))
    assert np.array_equal(c, np.array([[12.0, 16.0], [6.0, 8.0]], np.float32))


def _planted(N, K, seed):
    """Weights with a planted rank-8 part, and that part's noise alone (regenerated from the
    generator's definition: the bf16 weights minus nothing; see lowrank_weight_bits)."""
    return W.bits_to_f32(W.lowrank_weight_bits(N, K, seed)).astype(np.float64)


def test_residual_energy_meets_eckart_young_bound():
    """The rank-r residual is no larger than W minus any rank-r matrix: in particular at r = 8
    it is below the planted weights' noise part (W minus the planted rank-8 term), and it
    shrinks as r grows.  The factors' bf16 rounding adds at most ~2^-8 of the branch."""
    N, K, seed = 192, 128, 11
    w = _planted(N, K, seed)
    # the planted term, rebuilt from the generator's definition
    g1 = np.random.Generator(np.random.PCG64(seed + 1))
    g2 = np.random.Generator(np.random.PCG64(seed + 2))
    u = g1.standard_normal((N, 8), dtype=np.float32)
    v = g2.standard_normal((8, K), dtype=np.float32)
    gains = (8.0 * 2.0 ** (-0.5 * np.arange(8)) / np.sqrt(K)).astype(np.float32)
    planted = ((u * gains) @ v).astype(np.float64)
    noise = np.linalg.norm(w - planted)
    prev = None
    for r in (4, 8, 12, 16):
        l_up, l_down = S.factorize(w, r)
        res = np.linalg.norm(w - l_up @ l_down)
        slack = 2.0 ** -7 * np.linalg.norm(l_up @ l_down)
        if r >= 8:
            assert res <= noise + slack, (r, res, noise)
        if prev is not None:
            assert res <= prev + slack
        prev = res


def test_factors_are_orthonormal_directions():
    """L_down's rows are orthonormal and L_up's columns orthogonal, up to bf16 rounding."""
    w = _planted(160, 96, 5)
    l_up, l_down = S.factorize(w, 12)
    gram = l_down @ l_down.T
    assert np.max(np.abs(gram - np.eye(12))) < 2 ** -6
    gu = l_up.T @ l_up
    off = gu - np.diag(np.diag(gu))
    assert np.max(np.abs(off)) < 2 ** -6 * np.max(np.diag(gu))
    assert np.all(np.diff(np.diag(gu)) <= 2 ** -6 * np.max(np.diag(gu)))   # singular values fall


def test_branch_carries_the_planted_part():
    """With the branch the FP4 error is that of the small residual: against the exact bf16 GEMM
    A W^T the SVD-Quant output is several times closer than plain MXFP4 of W."""
    w = _planted(128, 256, 7).astype(np.float32)
    a = _acts(64, 256, 8)
    exact = a.astype(np.float64) @ w.astype(np.float64).T
    c0, _ = S.forward(a, *S.quantize_weights(w, 0)[:2], *S.quantize_weights(w, 0)[3:])
    l_up, l_down, _, rc, rs = S.quantize_weights(w, 16)
    c16, _ = S.forward(a, l_up, l_down, rc, rs)
    e0 = np.linalg.norm(c0 - exact) / np.linalg.norm(exact)
    e16 = np.linalg.norm(c16 - exact) / np.linalg.norm(exact)
    assert e16 < e0 / 2, (e0, e16)


# ---------------------------------------------------------------- planted mistakes

def _pins():
    return [test_rank_zero_is_the_mxfp4_gemm_of_the_weights, test_hand_worked_rank_one_case,
            test_residual_energy_meets_eckart_young_bound, test_factors_are_orthonormal_directions,
            test_branch_carries_the_planted_part]


def _caught():
    for pin in _pins():
        try:
            pin()
        except Exception:
            return True
    return False


def _factorize_one_more(w, rank):
    w = np.asarray(w, np.float64)
    U, s, Vt = np.linalg.svd(w, full_matrices=False)
    r = min(rank + 1, min(w.shape)) if rank else 0                       # planted: r + 1
    return S.bf16_round(U[:, :r] * s[:r]), S.bf16_round(Vt[:r])


def _factorize_smallest(w, rank):
    w = np.asarray(w, np.float64)
    U, s, Vt = np.linalg.svd(w, full_matrices=False)
    if rank == 0:
        return np.zeros((w.shape[0], 0)), np.zeros((0, w.shape[1]))
    return S.bf16_round(U[:, -rank:] * s[-rank:]), S.bf16_round(Vt[-rank:])   # planted: tail


_orig_forward = S.forward


def _forward_branch_dropped(a, l_up, l_down, rc, rs, branch=True):
    return _orig_forward(a, l_up, l_down, rc, rs, branch=False)            # planted


def _forward_branch_subtracted(a, l_up, l_down, rc, rs, branch=True):
    c, t = _orig_forward(a, l_up, l_down, rc, rs, branch=False)
    if branch and t.shape[1]:
        c = (c.astype(np.float64) - t @ l_up.T).astype(np.float32)         # planted: sign
    return c, t


_orig_residual = S.residual


def _residual_of_weights(w, l_up, l_down):
    return S.bf16_round(np.asarray(w, np.float64))                         # planted: no subtraction


@pytest.mark.parametrize("name,attr,fake", [
    ("rank truncated one too far", "factorize", _factorize_one_more),
    ("smallest singular values kept", "factorize", _factorize_smallest),
    ("16-bit branch dropped", "forward", _forward_branch_dropped),
    ("16-bit branch subtracted", "forward", _forward_branch_subtracted),
    ("residual not reduced by the branch", "residual", _residual_of_weights),
])
def test_planted_mistake_is_caught(monkeypatch, name, attr, fake):
    monkeypatch.setattr(S, attr, fake)
    assert _caught(), name
