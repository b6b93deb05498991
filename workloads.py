"""Seeded synthetic inputs for quantized attention at FLUX.1 Kontext shapes.

This module holds workload structure and random numbers only: tensor shapes,
the token composition of one Kontext sequence (text | target image | context
image), the integer 3-axis token positions, and seeded bf16 draws.  It holds
none of the quantized-attention arithmetic, so that both the CPU oracle and the
HIP path take their inputs from it without sharing any of the method's code.

Token layout (NVIDIA blog "Optimizing FLUX.1 Kontext for Image Editing with
Low-Precision Quantization", section "Workflow and Quantization": the input
image's tokens are concatenated with the output image's tokens, roughly doubling
the context; lpnh.cn "Flux.1 Kontext deep dive", sections 1 and 3: latents are
cut into 2x2 patches and concatenated along the sequence, target tokens sit at
positions (0, h, w) and context tokens at (i, h, w)).

Projection GEMMs (the linear layers around the attention): activations [M, K] with one row
per token (M = N of the sequence) and weights [N_out, K] with one row per output feature,
K = H * d = 3072; the QKV projection has N_out = 3 * 3072, the output projection 3072.
Activations ~ N(0, 1) with 1% outlier channels (x20) like Q, K, V, seed = seed; weights
~ N(0, 1/K), seed = seed + 1; both rounded to bf16.

Values: Q, K, V ~ N(0, 1) in float32 from numpy's PCG64 with
seed = 1000 * config_index + t (t = 0, 1, 2 for Q, K, V), optionally with 1% of
the H*d hidden channels (31 of 3072 at H=24, d=128; seed + 3 picks them) scaled
by 20 to mimic activation outliers, then rounded to bf16 (round to nearest
even, torch's CPU cast).  Arrays are returned as raw bf16 bit patterns
(numpy uint16), so both sides read identical bytes.
"""
from __future__ import annotations

import dataclasses
import functools

import numpy as np
import torch

__all__ = ["Workload", "CONFIGS", "config", "qkv_bits", "random_bits", "positions",
           "bits_to_f32", "GemmShape", "GEMM_SHAPES", "gemm_bits", "score_gap_bits",
           "lowrank_weight_bits", "PLANTED_RANK"]

OUTLIER_FRACTION = 0.01
OUTLIER_GAIN = 20.0


@dataclasses.dataclass(frozen=True)
class Workload:
    """One attention workload: shapes, token groups and quantization mode."""
    index: int              # 1-based config number; seeds derive from it
    name: str
    B: int
    H: int
    d: int
    n_text: int
    target_hw: tuple        # (rows, cols) of the target image's patch grid
    context_hw: tuple       # (rows, cols) of the context image's patch grid
    mode: str               # "fp8": per-tensor FP8 Q/K/V; "fp4": FP4 block quant then FP8
    rope: bool              # 3-axis rotary embedding on Q, K before FP4 quant
    outliers: bool

    @property
    def N(self) -> int:
        return (self.n_text + self.target_hw[0] * self.target_hw[1]
                + self.context_hw[0] * self.context_hw[1])

    @property
    def flops(self) -> int:
        """Dense attention work: 2*N*N*d for QK^T plus 2*N*N*d for P.V, per (b, h)."""
        return 4 * self.B * self.H * self.N * self.N * self.d


CONFIGS = [
    Workload(1, "tiny_sdpa_n256", 1, 2, 128, 64, (8, 12), (8, 12), "fp8", False, False),
    Workload(2, "kontext_512x512_n2560", 1, 24, 128, 512, (32, 32), (32, 32), "fp8", False, True),
    Workload(3, "kontext_1024x1024_n8704_fp8", 1, 24, 128, 512, (64, 64), (64, 64), "fp8", False,
             True),
    Workload(4, "kontext_1024x1024_n8704_fp4", 1, 24, 128, 512, (64, 64), (64, 64), "fp4", False,
             True),
    Workload(5, "multishape_b4_n4608_rope_fp4", 4, 24, 128, 512, (48, 64), (32, 32), "fp4", True,
             True),
]


def config(index_or_name) -> Workload:
    for c in CONFIGS:
        if c.index == index_or_name or c.name == index_or_name:
            return c
    raise KeyError(index_or_name)


def _to_bf16_bits(x: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> the float32 values they denote (exact)."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


def _draw(shape, seed: int) -> np.ndarray:
    return np.random.Generator(np.random.PCG64(seed)).standard_normal(shape, dtype=np.float32)


def _outlier_channels(H: int, d: int, seed: int) -> np.ndarray:
    n = max(1, int(OUTLIER_FRACTION * H * d))
    return np.random.Generator(np.random.PCG64(seed)).choice(H * d, size=n, replace=False)


def random_bits(B: int, H: int, N: int, d: int, seed: int, outliers: bool = False,
                scale: float = 1.0) -> np.ndarray:
    """bf16 bits of a [B, H, N, d] tensor ~ scale * N(0, 1), with optional outlier channels."""
    x = _draw((B, H, N, d), seed)
    if scale != 1.0:
        x *= np.float32(scale)
    if outliers:
        for c in _outlier_channels(H, d, seed + 3):
            x[:, c // d, :, c % d] *= np.float32(OUTLIER_GAIN)
    return _to_bf16_bits(x)


def score_gap_bits(H: int, N: int, gain: float, seed: int):
    """(q, k, v) bf16 bits [1, H, N, 128] whose score rows jump by a large power of two after the
    first key tiles: query rows are +1 (even rows) or -1 (odd rows) in every channel, plus
    N(0, 0.01^2) noise; keys 0..127 are N(0, 0.01^2), keys 128..191 are `gain` in every
    channel, the rest N(0, 1); values N(0, 1).  With gain 8 (16) the aligned keys score about
    130 (261) in the exp2 domain for the +1 rows and as far below for the -1 rows."""
    assert N > 192
    g = np.random.Generator(np.random.PCG64(seed))
    q = np.where((np.arange(N) % 2 == 0)[None, :, None], 1.0, -1.0).astype(np.float32)
    q = np.broadcast_to(q, (H, N, 128)) + 0.01 * g.standard_normal((H, N, 128), dtype=np.float32)
    k = g.standard_normal((H, N, 128), dtype=np.float32)
    k[:, :128] *= np.float32(0.01)
    k[:, 128:192] = np.float32(gain)
    v = g.standard_normal((H, N, 128), dtype=np.float32)
    return tuple(_to_bf16_bits(x[None]) for x in (q, k, v))


@functools.lru_cache(maxsize=3)
def qkv_bits(index: int):
    """(q, k, v) bf16 bit arrays [B, H, N, d] for config `index` (1-based)."""
    c = config(index)
    return tuple(random_bits(c.B, c.H, c.N, c.d, 1000 * c.index + t, c.outliers)
                 for t in range(3))


def positions(c: Workload) -> np.ndarray:
    """int32 [N, 3] token positions: text (0, 0, 0); target (0, h, w); context (1, h, w).

    Grids are row-major over (h, w).  A 1024 (wide) x 768 (tall) target image gives a
    48 x 64 grid of 2x2-patched latent tokens.
    """
    pos = np.zeros((c.N, 3), dtype=np.int32)
    o = c.n_text
    for image_index, (gh, gw) in ((0, c.target_hw), (1, c.context_hw)):
        hh, ww = np.meshgrid(np.arange(gh), np.arange(gw), indexing="ij")
        n = gh * gw
        pos[o:o + n, 0] = image_index
        pos[o:o + n, 1] = hh.reshape(-1)
        pos[o:o + n, 2] = ww.reshape(-1)
        o += n
    return pos


@dataclasses.dataclass(frozen=True)
class GemmShape:
    """One projection GEMM: C [M, N] = A [M, K] . W [N, K]^T."""
    name: str
    M: int
    N: int
    K: int

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K


GEMM_SHAPES = [
    GemmShape("kontext_1024_qkv_proj", 8704, 3 * 3072, 3072),
    GemmShape("kontext_1024_out_proj", 8704, 3072, 3072),
]


PLANTED_RANK = 8


def lowrank_weight_bits(N: int, K: int, seed: int, planted_rank: int = PLANTED_RANK,
                        gain: float = 8.0, cols=None):
    """bf16 bits of weights [N, K] with a planted low-rank outlier component, the structure the
    SVD-Quant branch is meant to absorb: N(0, 1/K) entries (seed) plus `planted_rank` rank-one
    terms g_i u_i v_i^T / sqrt(K), u_i ~ N(0, 1)^N, v_i ~ N(0, 1)^K (seed + 1, seed + 2), with
    g_i = gain * 2^(-i/2).  Each planted term's entries are ~g_i times the base spread.  `cols`
    (index array or None) selects output rows (weight rows) without changing their values."""
    w = _draw((N, K), seed) * np.float32(1.0 / np.sqrt(K))
    g1 = np.random.Generator(np.random.PCG64(seed + 1))
    g2 = np.random.Generator(np.random.PCG64(seed + 2))
    u = g1.standard_normal((N, planted_rank), dtype=np.float32)
    v = g2.standard_normal((planted_rank, K), dtype=np.float32)
    gains = (gain * 2.0 ** (-0.5 * np.arange(planted_rank)) / np.sqrt(K)).astype(np.float32)
    w = w + (u * gains) @ v
    if cols is not None:
        w = w[np.asarray(cols)]
    return _to_bf16_bits(w.astype(np.float32))


def gemm_bits(M: int, N: int, K: int, seed: int, rows=None, cols=None):
    """bf16 bits of (activations [M, K], weights [N, K]); `rows` / `cols` (index arrays or None)
    select rows of each without changing their values."""
    a = _draw((M, K), seed)
    n_out = max(1, int(OUTLIER_FRACTION * K))
    for c in np.random.Generator(np.random.PCG64(seed + 3)).choice(K, size=n_out, replace=False):
        a[:, c] *= np.float32(OUTLIER_GAIN)
    w = _draw((N, K), seed + 1) * np.float32(1.0 / np.sqrt(K))
    if rows is not None:
        a = a[np.asarray(rows)]
    if cols is not None:
        w = w[np.asarray(cols)]
    return _to_bf16_bits(a), _to_bf16_bits(w)
