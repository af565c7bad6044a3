"""Float64 reference for rotary position embedding (RoPE) at global
positions, with linear position interpolation.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Plain numpy.

Sources:
  [LL] PaperTrace "4.1.2 · LongLoRA: 用S²-Attn完成长上下文微调"
    §3.1 "位置外推与长内容学习如何分开": for one pair of channels RoPE at
      position m applies the plane rotation R(m, w) = [[cos mw, -sin mw],
      [sin mw, cos mw]], so (R(m)q)^T (R(n)k) = q^T R(n - m) k;
    §1.1 "Mask、位置与分布式边界": the rotation reads the token's original
      (global) position ID, never its offset inside a group -- the shift
      only permutes tensors; position interpolation maps a target position p
      to p * L0 / L1 before the angle is formed.

Readings of what the pages leave open (each tested as stated):
  * frequencies: pair i of a head of width D turns at w_i = base^(-2i/D),
    i = 0 .. D/2 - 1 (the pages name the rotation, not the schedule; this is
    the schedule of the Llama family the pages fine-tune), base a parameter;
  * pairing: HALF pairs channel i with channel i + D/2 (the layout of the
    Llama-2 checkpoints the pages use); INTERLEAVED pairs 2i with 2i + 1;
  * positions: int [B, N] position IDs, or 0 .. N-1 for every row when none
    are given; the angle of pair i at position p is (p * pos_scale) * w_i,
    with pos_scale = L0 / L1 for linear interpolation (1 for none);
  * the gradient of y = R x is x_bar = R^T y_bar (R is orthogonal).
"""
from __future__ import annotations

import numpy as np

HALF = 0
INTERLEAVED = 1


def frequencies(D: int, base: float) -> np.ndarray:
    """w_i = base^(-2i/D) for i = 0 .. D/2 - 1, float64."""
    if D <= 0 or D % 2:
        raise ValueError("D must be even and positive")
    i = np.arange(D // 2, dtype=np.float64)
    return np.float64(base) ** (-2.0 * i / D)


def positions(B: int, N: int, pos_ids=None) -> np.ndarray:
    """[B, N] float64 positions: the given IDs, else 0 .. N-1 per row."""
    if pos_ids is None:
        return np.broadcast_to(np.arange(N, dtype=np.float64), (B, N))
    p = np.asarray(pos_ids)
    if p.shape != (B, N):
        raise ValueError("pos_ids must be [B, N]")
    return p.astype(np.float64)


def pair_index(D: int, pairing: int):
    """(first, second) channel index arrays of the D/2 pairs."""
    i = np.arange(D // 2)
    if pairing == HALF:
        return i, i + D // 2
    if pairing == INTERLEAVED:
        return 2 * i, 2 * i + 1
    raise ValueError("pairing must be HALF or INTERLEAVED")


def rope(x, base: float = 10000.0, pos_scale: float = 1.0, pos_ids=None,
         pairing: int = HALF, inverse: bool = False) -> np.ndarray:
    """Rotate every pair of channels of x [B, N, H, D] by R(m, w_i) with
    m = position * pos_scale ([LL] §3.1; §1.1 for global positions and
    interpolation).  inverse=True applies R^T (the gradient map)."""
    x = np.asarray(x, dtype=np.float64)
    B, N, H, D = x.shape
    w = frequencies(D, base)
    m = positions(B, N, pos_ids) * np.float64(pos_scale)
    theta = m[:, :, None, None] * w[None, None, None, :]      # [B, N, 1, D/2]
    c, s = np.cos(theta), np.sin(theta)
    if inverse:
        s = -s
    a, b = pair_index(D, pairing)
    x1, x2 = x[..., a], x[..., b]
    y = np.empty_like(x)
    y[..., a] = c * x1 - s * x2
    y[..., b] = s * x1 + c * x2
    return y
