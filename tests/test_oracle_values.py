"""Pins of the oracle's forward / backward values.

Nothing here re-types the oracle's own formulas: values are checked against
an independent derivation (per-group attention after the layout change),
a library routine (torch's scaled_dot_product_attention in float64 on the
CPU), textbook causal attention brute-forced with Python loops, central
finite differences, and exact identities (slot-0 rows, padding invariance,
leak tests, log-sum-exp bounds, sum of dV).
"""
import math

import numpy as np
import pytest
import torch

import synthetic as syn
from oracle import (WRAP, SPLIT, CYCLIC, adjacency_block, backward,
                    backward_segments, forward, forward_segments,
                    group_maps_a, segments)


def rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


CASES = [  # B, N, H, D, G, L
    (1, 64, 4, 16, 16, 64),
    (2, 48, 4, 8, 12, 41),
    (1, 32, 2, 8, 8, 29),
    (1, 24, 2, 4, 24, 20),       # G = N
    (1, 40, 4, 8, 4, 40),
]


@pytest.mark.parametrize("B,N,H,D,G,L", CASES)
@pytest.mark.parametrize("boundary", [WRAP, SPLIT, CYCLIC])
@pytest.mark.parametrize("half", [0, 1])
def test_forward_two_derivations(B, N, H, D, G, L, boundary, half):
    q, k, v = (rand((B, N, H, D), s) for s in (1, 2, 3))
    sc = 1 / math.sqrt(D)
    shift = half * G // 2
    oa, la = forward(q, k, v, G, shift, boundary, L, sc)
    ob, lb = forward_segments(q, k, v, G, shift, boundary, L, sc)
    assert np.max(np.abs(oa - ob)) <= 1e-12
    fin = np.isfinite(la)
    assert np.array_equal(fin, np.isfinite(lb))
    assert np.max(np.abs(la[fin] - lb[fin])) <= 1e-12
    assert np.all(np.isneginf(la[:, :, L:])) and np.all(oa[:, L:] == 0)


@pytest.mark.parametrize("B,N,H,D,G,L", CASES)
@pytest.mark.parametrize("boundary", [WRAP, SPLIT, CYCLIC])
def test_backward_two_derivations(B, N, H, D, G, L, boundary):
    q, k, v, do = (rand((B, N, H, D), s) for s in (4, 5, 6, 7))
    do[:, L:] = 0
    sc = 1 / math.sqrt(D)
    dqa, dka, dva, oa, _ = backward(q, k, v, do, G, G // 2, boundary, L, sc)
    dqb, dkb, dvb = backward_segments(q, k, v, do, G, G // 2, boundary, L, sc)
    for x, y in ((dqa, dqb), (dka, dkb), (dva, dvb)):
        assert np.max(np.abs(x - y)) <= 1e-12
    for x in (dqa, dka, dva):
        assert np.all(x[:, L:] == 0)


@pytest.mark.parametrize("boundary", [WRAP, SPLIT, CYCLIC])
def test_unpadded_segments_match_library_sdpa(boundary):
    B, N, H, D, G = 1, 64, 4, 16, 16
    q, k, v = (rand((B, N, H, D), s) for s in (11, 12, 13))
    o, _ = forward(q, k, v, G, G // 2, boundary, N, 1 / math.sqrt(D))
    segs = segments(N, G, G // 2, boundary)
    for h in range(H):
        for pos in segs[int(h >= H // 2)]:
            t = [torch.from_numpy(np.ascontiguousarray(x[0, pos, h]))[None, None]
                 for x in (q, k, v)]
            ref = torch.nn.functional.scaled_dot_product_attention(
                *t, is_causal=True)[0, 0].numpy()
            assert np.max(np.abs(o[0, pos, h] - ref)) <= 1e-12


def _textbook_causal(q, k, v, sc):
    """Full causal softmax attention with explicit Python loops."""
    N, D = q.shape
    out = np.zeros((N, D))
    lse = np.zeros(N)
    for i in range(N):
        z = [sc * sum(q[i, d] * k[j, d] for d in range(D)) for j in range(i + 1)]
        m = max(z)
        w = [math.exp(x - m) for x in z]
        tot = sum(w)
        lse[i] = m + math.log(tot)
        for d in range(D):
            out[i, d] = sum(w[j] * v[j, d] for j in range(i + 1)) / tot
    return out, lse


@pytest.mark.parametrize("N", [4, 8, 12, 16])
@pytest.mark.parametrize("boundary", [WRAP, SPLIT, CYCLIC])
def test_g_equals_n_brute_force(N, boundary):
    B, H, D = 1, 2, 3
    q, k, v = (rand((B, N, H, D), s) for s in (21, 22, 23))
    sc = 1 / math.sqrt(D)
    o, lse = forward(q, k, v, N, N // 2, boundary, N, sc)
    for h in range(H):
        ro, rl = _textbook_causal(q[0, :, h], k[0, :, h], v[0, :, h], sc)
        assert np.max(np.abs(o[0, :, h] - ro)) <= 1e-12
        assert np.max(np.abs(lse[0, h] - rl)) <= 1e-12


@pytest.mark.parametrize("boundary", [WRAP, SPLIT, CYCLIC])
def test_slot0_rows_exact(boundary):
    """The first member of every group sees only itself: o = v exactly and
    lse = z_ii."""
    B, N, H, D, G, L = 1, 64, 4, 16, 16, 64
    q, k, v = (rand((B, N, H, D), s) for s in (31, 32, 33))
    sc = 1 / math.sqrt(D)
    o, lse = forward(q, k, v, G, G // 2, boundary, L, sc)
    _, slot, _ = group_maps_a(N, G, G // 2, boundary)
    for h in range(H):
        c = int(h >= H // 2)
        for x in np.nonzero(slot[c] == 0)[0]:
            assert np.array_equal(o[0, x, h], v[0, x, h])
            # equal up to the summation order of the dot product
            assert abs(lse[0, h, x] - sc * (q[0, x, h] @ k[0, x, h])) <= 1e-13


@pytest.mark.parametrize("boundary", [WRAP, SPLIT, CYCLIC])
def test_padding_invariance(boundary):
    """Changing padded rows of q, k, v leaves valid outputs bit-identical
    (padding never enters a softmax)."""
    B, N, H, D, G, L = 1, 64, 4, 8, 16, 45
    q, k, v, do = (rand((B, N, H, D), s) for s in (41, 42, 43, 44))
    do[:, L:] = 0
    sc = 1 / math.sqrt(D)
    o1, l1 = forward(q, k, v, G, G // 2, boundary, L, sc)
    g1 = backward(q, k, v, do, G, G // 2, boundary, L, sc)[:3]
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    for x in (q2, k2, v2):
        x[:, L:] = rand(x[:, L:].shape, 99) * 7
    o2, l2 = forward(q2, k2, v2, G, G // 2, boundary, L, sc)
    g2 = backward(q2, k2, v2, do, G, G // 2, boundary, L, sc)[:3]
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    for x, y in zip(g1, g2):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("boundary", [WRAP, SPLIT, CYCLIC])
def test_leak_perturb_key(boundary):
    """Editing k/v at position t changes exactly the rows whose visible set
    holds t.  Under SPLIT no row before t changes; under WRAP the rows < s
    change when t >= N - s (PaperTrace LongLoRA §1.1, packing leak test;
    §1, cyclic-shift paragraph)."""
    B, N, H, D, G, L = 1, 32, 2, 4, 8, 32
    s = G // 2
    q, k, v = (rand((B, N, H, D), s_) for s_ in (51, 52, 53))
    sc = 1 / math.sqrt(D)
    o1, _ = forward(q, k, v, G, s, boundary, L, sc)
    for t in (0, 3, 4, 13, N - s, N - 1):
        k2, v2 = k.copy(), v.copy()
        k2[0, t] += 1.0
        v2[0, t] -= 2.0
        o2, _ = forward(q, k2, v2, G, s, boundary, L, sc)
        for h in range(H):
            c = int(h >= H // 2)
            sees = adjacency_block(c, np.arange(N), N, G, s, boundary, L)[:, t]
            changed = np.any(o1[0, :, h] != o2[0, :, h], axis=1)
            assert np.array_equal(changed, sees)
            if c == 1 and boundary == SPLIT:
                assert not changed[:t].any()
            if c == 1 and boundary == WRAP and t >= N - s:
                assert changed[:s].all()


def test_lse_bounds_and_reconstruction():
    B, N, H, D, G, L = 1, 64, 4, 16, 16, 60
    q, k, v = (rand((B, N, H, D), s) for s in (61, 62, 63))
    sc = 1 / math.sqrt(D)
    for boundary in (WRAP, SPLIT):
        o, lse = forward(q, k, v, G, G // 2, boundary, L, sc)
        for h in range(H):
            c = int(h >= H // 2)
            a = adjacency_block(c, np.arange(N), N, G, G // 2, boundary, L)
            for i in range(L):
                js = np.nonzero(a[i])[0]
                z = sc * (k[0, js, h] @ q[0, i, h])
                assert z.max() - 1e-12 <= lse[0, h, i] <= z.max() + math.log(len(js)) + 1e-12
                rec = np.exp(z - lse[0, h, i]) @ v[0, js, h]
                assert np.max(np.abs(rec - o[0, i, h])) <= 1e-12


@pytest.mark.parametrize("boundary", [WRAP, SPLIT, CYCLIC])
@pytest.mark.parametrize("N,G,L", [(8, 4, 8), (8, 4, 5), (16, 4, 13), (12, 12, 12)])
def test_backward_finite_differences(boundary, N, G, L):
    B, H, D = 1, 2, 3
    q, k, v, do = (rand((B, N, H, D), s) for s in (71, 72, 73, 74))
    do[:, L:] = 0
    sc = 1 / math.sqrt(D)
    dq, dk, dv, _, _ = backward(q, k, v, do, G, G // 2, boundary, L, sc)

    def loss(q_, k_, v_):
        o, _ = forward(q_, k_, v_, G, G // 2, boundary, L, sc)
        return float(np.sum(do * o))

    h = 1e-6
    for name, grad in (("q", dq), ("k", dk), ("v", dv)):
        num = np.zeros_like(grad)
        for idx in np.ndindex(grad.shape):
            args = {"q": q.copy(), "k": k.copy(), "v": v.copy()}
            args[name][idx] += h
            lp = loss(args["q"], args["k"], args["v"])
            args[name][idx] -= 2 * h
            lm = loss(args["q"], args["k"], args["v"])
            num[idx] = (lp - lm) / (2 * h)
        err = np.max(np.abs(num - grad)) / max(1.0, np.max(np.abs(grad)))
        assert err < 1e-7, (name, err)


@pytest.mark.parametrize("boundary", [WRAP, SPLIT, CYCLIC])
def test_backward_invariants(boundary):
    B, N, H, D, G, L = 1, 64, 4, 8, 16, 57
    q, k, v, do = (rand((B, N, H, D), s) for s in (81, 82, 83, 84))
    do[:, L:] = 0
    sc = 1 / math.sqrt(D)
    dq, dk, dv, _, _ = backward(q, k, v, do, G, G // 2, boundary, L, sc)
    # softmax weights sum to one per row: sum_j dv_j = sum_{i<L} dO_i
    assert np.max(np.abs(dv.sum(axis=1) - do[:, :L].sum(axis=1))) <= 1e-11
    # a row that sees one key has no dq (up to summation order)
    _, slot, _ = group_maps_a(N, G, G // 2, boundary)
    for h in range(H):
        c = int(h >= H // 2)
        rows = [x for x in np.nonzero(slot[c] == 0)[0] if x < L]
        assert np.max(np.abs(dq[0, rows, h])) <= 1e-14
    # the sum over keys of dk is zero (sum_j dz_ij = 0)
    assert np.max(np.abs(dk.sum(axis=1))) <= 1e-11
    assert np.all(dq[:, L:] == 0) and np.all(dk[:, L:] == 0) and np.all(dv[:, L:] == 0)


def test_restricted_rows_match_full():
    """Computing one group's rows alone reproduces the full run on them."""
    B, N, H, D, G, L = 1, 64, 4, 8, 16, 64
    q, k, v, do = (rand((B, N, H, D), s) for s in (91, 92, 93, 94))
    sc = 1 / math.sqrt(D)
    full = backward(q, k, v, do, G, G // 2, WRAP, L, sc)
    gid, _, _ = group_maps_a(N, G, G // 2, WRAP)
    rows = np.nonzero(gid[1] == 3)[0]           # the wrapped group
    part = backward(q, k, v, do, G, G // 2, WRAP, L, sc, heads=[3], rows=rows)
    for t in range(3):
        assert np.max(np.abs(part[t][0, rows, 3] - full[t][0, rows, 3])) <= 1e-12


# ------------------------------------------------------------ document mask
def _docs(B, N, G, seed):
    # boundaries inside a group, on an original boundary and on a shifted one
    return syn.make_doc_ids(seed, B, N, mean_len=max(2, G // 2),
                            cuts=(G // 3, G, G + G // 2))


@pytest.mark.parametrize("boundary", [WRAP, SPLIT, CYCLIC])
@pytest.mark.parametrize("L", [48, 41])
def test_documents_two_derivations(boundary, L):
    B, N, H, D, G = 2, 48, 4, 8, 12
    q, k, v, do = (rand((B, N, H, D), s) for s in (91, 92, 93, 94))
    doc = _docs(B, N, G, 95)
    sc = 1 / math.sqrt(D)
    oa, la = forward(q, k, v, G, G // 2, boundary, L, sc, doc=doc)
    ob, lb = forward_segments(q, k, v, G, G // 2, boundary, L, sc, doc=doc)
    assert np.max(np.abs(oa - ob)) <= 1e-12
    fa, fb = np.isfinite(la), np.isfinite(lb)
    assert np.array_equal(fa, fb) and np.max(np.abs(la[fa] - lb[fb])) <= 1e-12
    ga = backward(q, k, v, do, G, G // 2, boundary, L, sc, doc=doc)[:3]
    gb = backward_segments(q, k, v, do, G, G // 2, boundary, L, sc, doc=doc)
    for x, y in zip(ga, gb):
        assert np.max(np.abs(x - y)) <= 1e-12


@pytest.mark.parametrize("boundary", [WRAP, SPLIT, CYCLIC])
def test_documents_leak(boundary):
    # [LL] §1.1: changing an earlier document must leave a later document's
    # outputs unchanged (boundaries inside a group and on both partitions'
    # boundaries)
    B, N, H, D, G, L = 1, 64, 4, 8, 16, 64
    q, k, v, do = (rand((B, N, H, D), s) for s in (101, 102, 103, 104))
    doc = _docs(B, N, G, 105)
    sc = 1 / math.sqrt(D)
    first = doc[0] == doc[0, 0]
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    for t in (q2, k2, v2):
        t[:, first] += rand(t[:, first].shape, 106)
    r1 = backward(q, k, v, do, G, G // 2, boundary, L, sc, doc=doc)
    r2 = backward(q2, k2, v2, do, G, G // 2, boundary, L, sc, doc=doc)
    later = ~first
    for x, y in zip(r1, r2):
        if x.ndim == 4:
            assert np.array_equal(x[:, later], y[:, later])
        else:
            assert np.array_equal(x[..., later], y[..., later])


def test_documents_special_cases():
    B, N, H, D, G, L = 1, 32, 2, 8, 8, 32
    q, k, v, do = (rand((B, N, H, D), s) for s in (111, 112, 113, 114))
    sc = 1 / math.sqrt(D)
    for boundary in (WRAP, SPLIT, CYCLIC):
        # one document: identical to no document mask
        one = np.zeros((B, N), np.int32)
        a = backward(q, k, v, do, G, G // 2, boundary, L, sc)
        b = backward(q, k, v, do, G, G // 2, boundary, L, sc, doc=one)
        for x, y in zip(a, b):
            assert np.array_equal(x, y)
        # one token per document: o = v, lse = scale q.k, no q/k gradient
        own = np.arange(N, dtype=np.int32)[None, :]
        dq, dk, dv, o, lse = backward(q, k, v, do, G, G // 2, boundary, L,
                                      sc, doc=own)
        assert np.max(np.abs(o - v)) <= 1e-15
        qk = np.einsum("bnhd,bnhd->bhn", q, k) * sc
        assert np.max(np.abs(lse - qk)) <= 1e-14
        # (zero up to the summation order of g.v against g.o)
        assert np.max(np.abs(dq)) <= 1e-14 and np.max(np.abs(dk)) <= 1e-14
        assert np.max(np.abs(dv - do)) <= 1e-15
