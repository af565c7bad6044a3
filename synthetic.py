"""Seeded synthetic inputs for S²-Attn workloads.

This module only draws numbers and names workload shapes.  It holds none of
the attention arithmetic, so both the float64 oracle's callers (tests,
cpu baseline) and the GPU path's callers (tests, bench) can use it without
the two sides sharing any code that decides a result.

Inputs are N(0,1) draws from numpy's PCG64 generator in float32, rounded
once to bfloat16 with round-to-nearest-even.  The GPU receives those bf16
bytes; the oracle receives the very same values widened to float64, so a
parity difference measures only the kernel's arithmetic.

Seed convention: ``1000*config + 10*variant + tensor`` with tensor index
q=0, k=1, v=2, dO=3.
"""
from __future__ import annotations

import math

import numpy as np

WRAP = 0
SPLIT = 1
CYCLIC = 2

# Workload shapes (Llama-2-7B attention layer: 32 heads of width 128).
# Each entry: B, N (padded length), H, D, list of G, list of boundary
# variants, valid length L, whether a backward pass is part of it.
WORKLOADS = {
    1: dict(name="tiny fwd B=1 N=64 H=4 D=16 G=16", B=1, N=64, H=4, D=16,
            Gs=[16], boundaries=[WRAP, SPLIT], L=64, bwd=False),
    2: dict(name="7B layer fwd B=1 N=8192 H=32 D=128 G=2048 split", B=1,
            N=8192, H=32, D=128, Gs=[2048], boundaries=[SPLIT], L=8192,
            bwd=False),
    3: dict(name="7B layer fwd+bwd B=1 N=32768 H=32 D=128 G=8192 wrap",
            B=1, N=32768, H=32, D=128, Gs=[8192], boundaries=[WRAP],
            L=32768, bwd=True),
    4: dict(name="ratio sweep B=2 N=12288 H=32 D=128 split", B=2, N=12288,
            H=32, D=128, Gs=[12288, 6144, 3072, 2048, 1536],
            boundaries=[SPLIT], L=12288, bwd=True),
    5: dict(name="ragged L=100000 padded N=102400 H=32 D=128 G=25600",
            B=1, N=102400, H=32, D=128, Gs=[25600],
            boundaries=[WRAP, SPLIT], L=100000, bwd=True),
}

TENSOR_INDEX = {"q": 0, "k": 1, "v": 2, "do": 3}


def seed_for(config: int, variant: int, tensor: str) -> int:
    return 1000 * config + 10 * variant + TENSOR_INDEX[tensor]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return the
    16-bit patterns as uint16.  Inputs here are finite normal draws."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(bits).astype(np.float64)


def normal_f32(seed: int, shape) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(seed))
    return g.standard_normal(size=shape, dtype=np.float32)


def normal_bf16_bits(seed: int, shape) -> np.ndarray:
    """N(0,1) float32 draws rounded to bf16, as uint16 bit patterns."""
    return f32_to_bf16_bits(normal_f32(seed, shape))


def make_inputs(config: int, variant: int, B: int, N: int, H: int, D: int,
                with_do: bool = False, L: int | None = None) -> dict:
    """q, k, v (and dO) as bf16 bit patterns of shape [B,N,H,D].

    Every row, padded ones included, gets random values so that a missing
    padding mask shows up as a wrong result.  dO rows at positions >= L are
    set to zero (the loss mask of a padded tail)."""
    shape = (B, N, H, D)
    out = {t: normal_bf16_bits(seed_for(config, variant, t), shape)
           for t in ("q", "k", "v")}
    if with_do:
        do = normal_bf16_bits(seed_for(config, variant, "do"), shape)
        if L is not None and L < N:
            do[:, L:] = 0
        out["do"] = do
    return out


def make_doc_ids(seed: int, B: int, N: int, mean_len: int,
                 cuts=()) -> np.ndarray:
    """Packed-sequence document IDs, int32 [B, N], non-decreasing along each
    row: document lengths are drawn from a geometric distribution with the
    given mean (a mix of short and long samples), and every position in
    ``cuts`` additionally starts a new document (to place boundaries inside
    a group, on an original group boundary or on a shifted one)."""
    g = np.random.Generator(np.random.PCG64(seed))
    out = np.empty((B, N), np.int32)
    for b in range(B):
        starts = np.zeros(N, bool)
        x = 0
        while x < N:
            starts[x] = True
            x += int(g.geometric(1.0 / max(1, mean_len)))
        for c in cuts:
            if 0 <= c < N:
                starts[c] = True
        out[b] = np.cumsum(starts) - 1
    return out


def doc_positions(doc: np.ndarray) -> np.ndarray:
    """Position IDs of packed samples: int32 [B, N], restarting at 0 where
    the document ID changes (each packed sample keeps its own positions)."""
    doc = np.asarray(doc)
    B, N = doc.shape
    out = np.empty((B, N), np.int32)
    for b in range(B):
        start = 0
        for x in range(N):
            if x and doc[b, x] != doc[b, x - 1]:
                start = x
            out[b, x] = x - start
    return out


def default_scale(D: int) -> float:
    return 1.0 / math.sqrt(D)
