"""Pins of the oracle's group maps and edge sets against what the pages fix.

Worked examples are read from tests/golden/worked_examples.json (each entry
carries its citation).  Closed-form pair counts are written out from the
complexity paragraph of PaperTrace "4.1.2 · LongLoRA: 用S²-Attn完成长上下文微调"
§1; the brute-force visible sets are built with plain Python lists by
rolling / splitting a list of positions, independently of the oracle.
"""
import json
import os

import numpy as np
import pytest

from oracle import (WRAP, SPLIT, CYCLIC, OracleError, adjacency_block,
                    adjacency_dense, allowed_pairs, group_maps_a,
                    group_maps_b, segments, validate)

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                   "worked_examples.json")))


def visible(cls, i, N, G, boundary, L=None, shift=None):
    L = N if L is None else L
    shift = G // 2 if shift is None else shift
    row = adjacency_block(cls, np.array([i]), N, G, shift, boundary, L)[0]
    return sorted(np.nonzero(row)[0].tolist())


# ----------------------------------------------------------------- N=8, G=4
def test_n8_unshifted_groups():
    ex = GOLD["n8_g4"]
    segs = segments(ex["N"], ex["G"], ex["G"] // 2, WRAP)[0]
    assert [s.tolist() for s in segs] == ex["unshifted_groups"]
    gid, slot, _ = group_maps_a(ex["N"], ex["G"], ex["G"] // 2, SPLIT)
    for g, grp in enumerate(ex["unshifted_groups"]):
        for j, x in enumerate(grp):
            assert gid[0, x] == g and slot[0, x] == j


@pytest.mark.parametrize("boundary", [WRAP, SPLIT])
def test_n8_shifted_middle_group(boundary):
    ex = GOLD["n8_g4"]
    N, G = ex["N"], ex["G"]
    gid, slot, _ = group_maps_a(N, G, G // 2, boundary)
    mid = ex["shifted_middle_group"]
    g = gid[1, mid[0]]
    assert all(gid[1, x] == g for x in mid)
    assert sorted(np.nonzero(gid[1] == g)[0].tolist()) == mid
    assert [slot[1, x] for x in mid] == [0, 1, 2, 3]
    assert any(s.tolist() == mid for s in segments(N, G, G // 2, boundary)[1])


@pytest.mark.parametrize("boundary", [WRAP, SPLIT])
def test_n8_position4_visible_sets(boundary):
    ex = GOLD["n8_g4"]
    N, G = ex["N"], ex["G"]
    assert visible(0, 4, N, G, boundary) == ex["visible_from_4_unshifted"]
    assert visible(1, 4, N, G, boundary) == ex["visible_from_4_shifted"]


def test_n8_wrapped_group():
    ex = GOLD["n8_g4"]
    N, G = ex["N"], ex["G"]
    s = G // 2
    gid, slot, src = group_maps_a(N, G, s, WRAP)
    last = ex["wrap_last_group_in_rolled_order"]
    assert src[1, N - G:].tolist() == last
    assert segments(N, G, s, WRAP)[1][-1].tolist() == last
    assert [slot[1, x] for x in last] == list(range(G))
    assert all(gid[1, x] == N // G - 1 for x in last)
    # the wrapped triangle lets position 0 read 6 and 7 (plus itself)
    v0 = visible(1, 0, N, G, WRAP)
    assert set(ex["wrap_position_0_reads"]) <= set(v0)
    assert v0 == sorted(ex["wrap_position_0_reads"] + [0])
    # the strict-causal split keeps it to itself
    assert visible(1, 0, N, G, SPLIT) == [0]
    segs = segments(N, G, s, SPLIT)[1]
    assert [x.tolist() for x in segs] == [[0, 1], [2, 3, 4, 5], [6, 7]]


# ---------------------------------------------------------------- N=16, G=4
@pytest.mark.parametrize("boundary", [WRAP, SPLIT])
def test_n16_visible_sets(boundary):
    ex = GOLD["n16_g4"]
    N, G = ex["N"], ex["G"]
    assert ex["s"] == G // 2
    for q, want in ex["visible_unshifted"].items():
        assert visible(0, int(q), N, G, boundary) == want
    for q, want in ex["visible_shifted"].items():
        assert visible(1, int(q), N, G, boundary) == want


# ------------------------------------------------------------ N=8192, G=2048
@pytest.mark.parametrize("boundary", [WRAP, SPLIT])
def test_n8192_group_bounds(boundary):
    ex = GOLD["n8192_g2048"]
    N, G = ex["N"], ex["G"]
    gid, slot, _ = group_maps_a(N, G, G // 2, boundary)

    def members(c, g):
        m = np.nonzero(gid[c] == g)[0]
        return [int(m.min()) + 1, int(m.max()) + 1]   # 1-based bounds

    assert members(0, 0) == ex["pattern1_first_group_1based"]
    assert members(0, 1) == ex["pattern1_second_group_1based"]
    first_full = 0 if boundary == WRAP else 1   # SPLIT: group 0 is the short head
    assert members(1, first_full) == ex["pattern2_first_group_1based"]
    assert members(1, first_full + 1) == ex["pattern2_second_group_1based"]


# ---------------------------------------------- two derivations of the maps
MAP_CASES = [(8, 4), (16, 4), (64, 16), (48, 12), (12, 12), (24, 2),
             (8192, 2048), (32768, 8192), (12288, 1536), (12288, 12288),
             (102400, 25600)]


@pytest.mark.parametrize("N,G", MAP_CASES)
@pytest.mark.parametrize("boundary", [WRAP, SPLIT, CYCLIC])
@pytest.mark.parametrize("half", [0, 1])
def test_maps_a_equal_b(N, G, boundary, half):
    shift = half * G // 2
    a = group_maps_a(N, G, shift, boundary)
    b = group_maps_b(N, G, shift, boundary)
    for x, y in zip(a, b):
        assert x.dtype == np.int32 and y.dtype == np.int32
        assert np.array_equal(x, y)


def _brute_sets(cls, N, G, boundary, L):
    """Visible sets built with lists: roll or split a list of positions,
    chunk it, and give each member the members at or before it in chunk
    order, keeping valid positions only."""
    s = G // 2 if (cls == 1 and N // G > 1) else 0
    pos = list(range(N))
    if s == 0:
        chunks = [pos[t:t + G] for t in range(0, N, G)]
    elif boundary in (WRAP, CYCLIC):
        rolled = pos[s:] + pos[:s]
        chunks = [rolled[t:t + G] for t in range(0, N, G)]
        if boundary == CYCLIC:       # causal order = original order
            chunks = [sorted(ch) for ch in chunks]
    else:
        cuts = [0, s] + [s + t * G for t in range(1, N // G)] + [N]
        chunks = [pos[a:b] for a, b in zip(cuts[:-1], cuts[1:])]
    sets = {}
    for ch in chunks:
        for r, i in enumerate(ch):
            sets[i] = sorted(j for j in ch[:r + 1] if j < L) if i < L else []
    return [sets[i] for i in range(N)]


@pytest.mark.parametrize("N,G", [(8, 4), (16, 4), (24, 6), (12, 12), (20, 4),
                                 (32, 8)])
@pytest.mark.parametrize("boundary", [WRAP, SPLIT, CYCLIC])
@pytest.mark.parametrize("L", [1, 3, 4, 5, 7, 8, None])
def test_adjacency_brute_force(N, G, boundary, L):
    """Validation lengths 1,3,4,5,7,8 cover partial groups (PaperTrace
    LongLoRA §1.1, FP64 small-shape validation paragraph)."""
    L = N if L is None else min(L, N)
    for cls in (0, 1):
        a = adjacency_dense(cls, N, G, G // 2, boundary, L)
        want = _brute_sets(cls, N, G, boundary, L)
        got = [sorted(np.nonzero(a[i])[0].tolist()) for i in range(N)]
        assert got == want


# ----------------------------------------------------- closed-form counts
@pytest.mark.parametrize("N,G", [(64, 16), (48, 12), (256, 64), (4096, 1024),
                                 (3072, 512), (12, 12), (4096, 4096)])
def test_pair_counts_closed_form(N, G):
    M = N // G
    s = G // 2 if M > 1 else 0
    per_group = G * (G + 1) // 2
    c0 = M * per_group                           # M*G*(G+1)/2
    wrap1 = M * per_group
    split1 = (M - 1) * per_group + s * (s + 1) if s else c0
    assert allowed_pairs(N, G, G // 2, WRAP, N) == (c0, wrap1)
    assert allowed_pairs(N, G, G // 2, SPLIT, N) == (c0, split1)
    # the cyclic-causal graph keeps WRAP's partition, so its triangles too
    assert allowed_pairs(N, G, G // 2, CYCLIC, N) == (c0, wrap1)
    if M > 1:
        # WRAP adds exactly s*s edges: queries 0..s-1 reading keys N-s..N-1
        assert wrap1 - split1 == s * s


def test_pair_ratio_tends_to_g_over_n():
    # the per-head ratio to full causal N(N+1)/2 approaches G/N
    for N, G in [(4096, 1024), (8192, 1024), (4096, 512)]:
        c0, c1 = allowed_pairs(N, G, G // 2, WRAP, N)
        ratio = (c0 + c1) / 2 / (N * (N + 1) / 2)
        assert abs(ratio - G / N) < 2.0 / G


# ------------------------------------------------------------- invariants
@pytest.mark.parametrize("N,G,L", [(64, 16, 64), (64, 16, 50), (48, 12, 37),
                                   (96, 32, 96), (96, 32, 70)])
def test_adjacency_invariants(N, G, L):
    s = G // 2
    for boundary in (WRAP, SPLIT):
        a0 = adjacency_dense(0, N, G, s, boundary, L)
        a1 = adjacency_dense(1, N, G, s, boundary, L)
        tril = np.tril(np.ones((N, N), bool))
        valid = np.arange(N) < L
        for a in (a0, a1):
            assert np.array_equal(np.diag(a), valid)      # (i, i) allowed
            assert not a[~valid].any() and not a[:, ~valid].any()
        assert not (a0 & ~tril).any()
        if boundary == SPLIT:
            assert not (a1 & ~tril).any()
    w = adjacency_dense(1, N, G, s, WRAP, L)
    sp = adjacency_dense(1, N, G, s, SPLIT, L)
    assert not (sp & ~w).any()
    extra = np.zeros((N, N), bool)
    extra[:s, N - s:] = True
    valid = np.arange(N) < L
    extra &= valid[:, None] & valid[None, :]
    assert np.array_equal(w & ~sp, extra)
    # cyclic-causal: no edge points to a later position; its s*s extra
    # edges over SPLIT are the tail N-s..N-1 reading the head 0..s-1, the
    # transpose of WRAP's, so the two modes share exactly SPLIT's edges
    cy = adjacency_dense(1, N, G, s, CYCLIC, L)
    tril = np.tril(np.ones((N, N), bool))
    assert not (cy & ~tril).any()
    assert not (sp & ~cy).any()
    back = np.zeros((N, N), bool)
    back[N - s:, :s] = True
    back &= valid[:, None] & valid[None, :]
    assert np.array_equal(cy & ~sp, back)
    assert np.array_equal(cy & w, sp)


def test_g_equals_n_is_full_causal():
    for N in (4, 8, 12, 16):
        for boundary in (WRAP, SPLIT, CYCLIC):
            for cls in (0, 1):
                a = adjacency_dense(cls, N, N, N // 2, boundary, N)
                assert np.array_equal(a, np.tril(np.ones((N, N), bool)))


def test_shift_zero_both_classes_equal():
    for boundary in (WRAP, SPLIT, CYCLIC):
        a0 = adjacency_dense(0, 64, 16, 0, boundary, 64)
        a1 = adjacency_dense(1, 64, 16, 0, boundary, 64)
        assert np.array_equal(a0, a1)
        g, sl, sr = group_maps_a(64, 16, 0, boundary)
        assert np.array_equal(g[0], g[1]) and np.array_equal(sl[0], sl[1])


@pytest.mark.parametrize("args", [
    dict(N=64, H=3, D=16, G=16, shift=8, boundary=WRAP, L=64),
    dict(N=64, H=4, D=16, G=15, shift=7, boundary=WRAP, L=60),
    dict(N=60, H=4, D=16, G=16, shift=8, boundary=WRAP, L=60),
    dict(N=64, H=4, D=16, G=16, shift=4, boundary=WRAP, L=64),
    dict(N=64, H=4, D=16, G=16, shift=8, boundary=3, L=64),
    dict(N=64, H=4, D=16, G=16, shift=8, boundary=WRAP, L=0),
    dict(N=64, H=4, D=16, G=16, shift=8, boundary=WRAP, L=65),
])
def test_validate_rejects(args):
    with pytest.raises(OracleError):
        validate(**args)
