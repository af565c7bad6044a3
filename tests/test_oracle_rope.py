"""Pins of the float64 RoPE reference (oracle/rope.py) against the rotation
the pages print ([LL] §3.1), closed forms and invariants -- never against
its own formula typed again."""
import math

import numpy as np
import pytest

from oracle import HALF, INTERLEAVED, frequencies, rope


def rand(shape, seed):
    return np.random.Generator(np.random.PCG64(seed)).standard_normal(shape)


@pytest.mark.parametrize("m", [0, 1, 2, 7, 1000, -3])
def test_one_pair_is_the_printed_rotation(m):
    # D = 2 is one pair with w_0 = 1: R(m) applied to the unit vectors
    # gives the columns of [[cos m, -sin m], [sin m, cos m]] ([LL] §3.1).
    e1 = np.array([1.0, 0.0]).reshape(1, 1, 1, 2)
    e2 = np.array([0.0, 1.0]).reshape(1, 1, 1, 2)
    pos = np.array([[m]])
    for pairing in (HALF, INTERLEAVED):
        c1 = rope(e1, pos_ids=pos, pairing=pairing).ravel()
        c2 = rope(e2, pos_ids=pos, pairing=pairing).ravel()
        assert np.allclose(c1, [math.cos(m), math.sin(m)], rtol=0, atol=1e-15)
        assert np.allclose(c2, [-math.sin(m), math.cos(m)], rtol=0, atol=1e-15)


def test_frequency_schedule_closed_form():
    # base 100, D = 8: w_i = 100^(-2i/8) = 10^(-i/2)
    want = [1.0, 0.31622776601683794, 0.1, 0.031622776601683794]
    assert np.allclose(frequencies(8, 100.0), want, rtol=1e-15, atol=0)
    # and the rotation of pair i at position m turns by m * w_i
    m = 3
    for i, wi in enumerate(want):
        x = np.zeros((1, 1, 1, 8))
        x[..., i] = 1.0                      # HALF: pair (i, i + 4)
        y = rope(x, base=100.0, pos_ids=np.array([[m]])).ravel()
        assert abs(y[i] - math.cos(m * wi)) < 1e-15
        assert abs(y[i + 4] - math.sin(m * wi)) < 1e-15
        assert np.count_nonzero(np.abs(y) > 1e-300) == 2


def test_pairings_touch_the_stated_channels():
    D = 8
    pos = np.array([[5]])
    x = np.zeros((1, 1, 1, D))
    x[..., 1] = 1.0
    y = rope(x, pos_ids=pos, pairing=HALF).ravel()
    assert set(np.flatnonzero(y)) == {1, 5}
    x = np.zeros((1, 1, 1, D))
    x[..., 2] = 1.0
    y = rope(x, pos_ids=pos, pairing=INTERLEAVED).ravel()
    assert set(np.flatnonzero(y)) == {2, 3}


@pytest.mark.parametrize("pairing", [HALF, INTERLEAVED])
def test_relative_position_identity(pairing):
    # (R(m) q)^T (R(n) k) = q^T R(n - m) k  ([LL] §3.1)
    D = 16
    q = rand((1, 1, 1, D), 1)
    k = rand((1, 1, 1, D), 2)
    for m, n in [(0, 0), (3, 11), (11, 3), (4000, 4093), (32767, 5)]:
        lhs = np.sum(rope(q, pos_ids=np.array([[m]]), pairing=pairing) *
                     rope(k, pos_ids=np.array([[n]]), pairing=pairing))
        rhs = np.sum(q * rope(k, pos_ids=np.array([[n - m]]), pairing=pairing))
        assert abs(lhs - rhs) <= 1e-11 * max(1.0, abs(lhs))


@pytest.mark.parametrize("pairing", [HALF, INTERLEAVED])
def test_orthogonal_identity_at_zero_and_adjoint(pairing):
    B, N, H, D = 2, 9, 3, 32
    x = rand((B, N, H, D), 3)
    y = rand((B, N, H, D), 4)
    pos = np.random.Generator(np.random.PCG64(5)).integers(-50, 100000, (B, N))
    rx = rope(x, base=500000.0, pos_ids=pos, pairing=pairing)
    # norms of every pair are kept, so the whole row norm is too
    assert np.allclose(np.linalg.norm(rx, axis=-1), np.linalg.norm(x, axis=-1),
                       rtol=1e-13, atol=0)
    # R^T R = I
    back = rope(rx, base=500000.0, pos_ids=pos, pairing=pairing, inverse=True)
    assert np.max(np.abs(back - x)) <= 1e-12
    # <R x, y> = <x, R^T y>: the inverse map is the gradient map
    lhs = np.sum(rx * y)
    rhs = np.sum(x * rope(y, base=500000.0, pos_ids=pos, pairing=pairing,
                          inverse=True))
    assert abs(lhs - rhs) <= 1e-10 * np.sum(np.abs(x * y))
    # position 0 is the identity
    z = rope(x, pos_ids=np.zeros((B, N), np.int64), pairing=pairing)
    assert np.array_equal(z, x)


def test_default_positions_are_global_indices():
    B, N, H, D = 2, 40, 2, 8
    x = rand((B, N, H, D), 6)
    a = rope(x)
    b = rope(x, pos_ids=np.tile(np.arange(N), (B, 1)))
    assert np.array_equal(a, b)
    # a row's result depends on its own position only: rows of a batch with
    # permuted position IDs are the same rows, permuted
    perm = np.random.Generator(np.random.PCG64(7)).permutation(N)
    c = rope(x[:, perm], pos_ids=np.tile(perm, (B, 1)))
    assert np.array_equal(c, a[:, perm])


def test_position_interpolation():
    # p * L0 / L1: interpolating by 1/4 equals rotating at p / 4 ([LL] §1.1)
    B, N, H, D = 1, 64, 2, 16
    x = rand((B, N, H, D), 8)
    pos = np.tile(np.arange(0, 4 * N, 4), (B, 1))
    a = rope(x, pos_ids=pos, pos_scale=0.25)
    b = rope(x, pos_ids=pos // 4)
    assert np.array_equal(a, b)


def test_logits_invariant_to_a_global_position_offset():
    # logits depend on position differences only: the attention pattern of
    # any group is unchanged when every position ID moves by the same amount
    B, N, H, D = 1, 48, 2, 16
    q, k = rand((B, N, H, D), 9), rand((B, N, H, D), 10)
    pos = np.tile(np.arange(N), (B, 1))
    s0 = np.einsum("bihd,bjhd->bhij", rope(q, pos_ids=pos), rope(k, pos_ids=pos))
    s1 = np.einsum("bihd,bjhd->bhij", rope(q, pos_ids=pos + 12345),
                   rope(k, pos_ids=pos + 12345))
    assert np.max(np.abs(s0 - s1)) <= 1e-10


def test_group_local_offsets_would_differ():
    # Inside an unwrapped group, in-group offsets are global positions minus
    # a constant, so by the identity above they give the same logits.  In
    # the wrapped group of the original roll they do not: for N = 16, G = 8
    # the shifted class's last group holds positions 12..15, 0..3, so query
    # 0 (offset 4) and key 15 (offset 3) are 1 apart in offsets but -15
    # apart globally -- the mistake [LL] §1.1 warns about.
    D = 16
    q, k = rand((1, 1, 1, D), 11), rand((1, 1, 1, D), 12)

    def logit(mq, mk):
        return np.sum(rope(q, pos_ids=np.array([[mq]])) *
                      rope(k, pos_ids=np.array([[mk]])))

    assert abs(logit(9, 6) - logit(9 - 4, 6 - 4)) <= 1e-12   # group [4, 12)
    assert abs(logit(0, 15) - logit(4, 3)) > 1e-3
