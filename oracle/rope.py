"""3-axis rotary position embedding applied to Q and K before FP4 quantization.

lpnh.cn "Flux.1 Kontext deep dive", sections 1 and 3: target-image tokens carry
positions (0, h, w) and context-image tokens (i, h, w); the sequence is the
length-wise concatenation of the token groups.  The pages give no formula, so
the plainest reading is the standard rotary embedding applied per axis:

  * the head dimension d = 128 is cut into consecutive axis slices of widths
    (16, 56, 56) for the position axes (index, h, w); text tokens sit at (0, 0, 0)
    and the context image uses index i = 1;
  * within axis a of width d_a, pair k (k < d_a/2) turns by angle
    pos_a * w_k with w_k = 1 / theta^(2k/d_a), theta = 10000;
  * adjacent elements (x[2j], x[2j+1]) form pair j of the head dimension;
  * the angle and its cos/sin are evaluated in float64 and stored as float32;
  * the rotation is (x0, x1) -> (fl32(fl32(x0 c) - fl32(x1 s)), fl32(fl32(x0 s) + fl32(x1 c)))
    with every product and sum rounded to float32 separately (no fused multiply-add).
V is not rotated.
"""
from __future__ import annotations

import math

import numpy as np

AXES = (16, 56, 56)
THETA = 10000.0


def table(pos, axes=AXES, theta: float = THETA) -> np.ndarray:
    """float32 [N, d/2, 2] table of (cos, sin) for integer positions pos [N, len(axes)]."""
    pos = np.asarray(pos)
    n_pairs = sum(axes) // 2
    out = np.empty((pos.shape[0], n_pairs, 2), dtype=np.float32)
    for n in range(pos.shape[0]):
        j = 0
        for a, d_a in enumerate(axes):
            p = float(pos[n, a])
            for k in range(d_a // 2):
                w = 1.0 / math.pow(theta, (2.0 * k) / d_a)
                ang = p * w
                out[n, j, 0] = math.cos(ang)
                out[n, j, 1] = math.sin(ang)
                j += 1
    return out


def apply(x_f32, tab) -> np.ndarray:
    """Rotate adjacent pairs of x [..., N, d] (float32) by the table [N, d/2, 2]."""
    x = np.asarray(x_f32, dtype=np.float32)
    c = tab[:, :, 0]
    s = tab[:, :, 1]
    x0 = x[..., 0::2]
    x1 = x[..., 1::2]
    y = np.empty_like(x)
    y[..., 0::2] = (x0 * c) - (x1 * s)          # numpy float32: each op rounds separately
    y[..., 1::2] = (x0 * s) + (x1 * c)
    return y
