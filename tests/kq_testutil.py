"""Shared helpers for the GPU parity tests (device transfer, row sampling, error metrics)."""
import numpy as np
import torch

REL_L2_TOL = 1e-2
MAX_ABS_TOL = 5e-2


def to_dev(bits: np.ndarray) -> torch.Tensor:
    """bf16 device tensor with the given bit patterns."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def rel_l2(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / nb) if nb > 0 else float(np.linalg.norm(a - b))


def max_abs(a, b) -> float:
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64))))


def sample_rows(N: int, n_random: int, seed: int) -> np.ndarray:
    """Query rows to compare at full size: the edges of every token group boundary the
    workloads use, the last row, and seeded random rows."""
    fixed = [0, 1, 63, 64, 127, 128, 511, 512, 513, N // 2, N - 129, N - 128, N - 2, N - 1]
    rng = np.random.default_rng(seed)
    rnd = rng.choice(N, size=min(n_random, N), replace=False)
    rows = np.unique(np.clip(np.concatenate([fixed, rnd]), 0, N - 1))
    return rows.astype(np.int64)


def all_finite_bf16_rows(d: int = 128, seed: int = 0) -> np.ndarray:
    """Every finite bf16 bit pattern once, shuffled and padded with zeros to rows of d."""
    bits = np.arange(1 << 16, dtype=np.uint32)
    bits = bits[((bits >> 7) & 0xFF) != 0xFF].astype(np.uint16)
    bits = np.random.default_rng(seed).permutation(bits)
    pad = (-len(bits)) % d
    return np.concatenate([bits, np.zeros(pad, np.uint16)]).reshape(-1, d)
