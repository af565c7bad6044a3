"""CPU checks of the sequence-parallel shard calls: the halo that
s2attn_shard_halo names is exactly the set of keys outside a slice that the
slice's valid queries read, as the oracle's adjacency of the shifted heads
says ([LL] §1.1, the paragraphs on sequence-parallel communication: with
slice edges on the unshifted groups' edges only the shifted heads cross
them), and bad shard arguments are rejected before any launch."""
import ctypes

import numpy as np
import pytest

import oracle
from sparse_attention_long_attn_amd import _lib, work

BOUNDS = (oracle.WRAP, oracle.SPLIT, oracle.CYCLIC)


def halo(N, row0, T, G, shift, boundary, L):
    lib = _lib.load()
    out = [ctypes.c_int(-7) for _ in range(3)]
    st = lib.s2attn_shard_halo(N, row0, T, G, shift, boundary, L,
                               *(ctypes.byref(o) for o in out))
    assert st == _lib.S2A_OK, lib.s2attn_last_error()
    return tuple(o.value for o in out)


def read_across(N, G, shift, boundary, L, row0, T):
    """Oracle: (keys read across the slice's left edge, keys read across
    the wrap).  With several slices these are the keys outside the slice
    that its queries read, split by side; with one slice (all rows), the
    keys that queries 0..s-1 read from the end of the sequence and that
    queries N-s..N-1 read from its start."""
    s = oracle.effective_shift(N, G, shift)
    rows = np.arange(row0, row0 + T)
    a = oracle.adjacency_block(1, rows, N, G, shift, boundary, L)
    a0 = oracle.adjacency_block(0, rows, N, G, shift, boundary, L)
    inside = (np.arange(N) >= row0) & (np.arange(N) < row0 + T)
    # the unshifted class never leaves its slice
    assert not np.any(a0[:, ~inside])
    if T < N:
        outside = np.flatnonzero(~inside)
        seen = outside[np.any(a[:, outside], axis=0)]
        # left: the s rows just before row0, cyclically
        left = {int(y) for y in seen if 1 <= (row0 - y) % N <= s}
        wrap = {int(y) for y in seen} - left
        return left, wrap
    if s == 0:
        return set(), set()
    head, tail = a[:s], a[N - s:]
    left = {int(y) + s for y in np.flatnonzero(np.any(head[:, s:], axis=0))}
    wrap = {int(y) for y in np.flatnonzero(np.any(tail[:, :N - s], axis=0))}
    return left, wrap


@pytest.mark.parametrize("boundary", BOUNDS)
@pytest.mark.parametrize("N,G,P", [(64, 16, 1), (64, 16, 2), (64, 16, 4),
                                   (96, 16, 3), (64, 32, 2), (32, 32, 1),
                                   (48, 8, 6)])
@pytest.mark.parametrize("pad", [0, 1, 5, 8, 20, 40])
@pytest.mark.parametrize("half", [1, 0])
def test_halo_is_what_the_slice_reads(boundary, N, G, P, pad, half):
    L = N - pad
    if L < 1:
        return
    shift = half * G // 2
    s = oracle.effective_shift(N, G, shift)
    T = N // P
    for r in range(P):
        row0 = r * T
        left0, hl, hw = halo(N, row0, T, G, shift, boundary, L)
        want_left, want_wrap = read_across(N, G, shift, boundary, L, row0, T)
        assert set(range(left0, left0 + hl)) == want_left, (r, left0, hl)
        assert set(range(hw)) == want_wrap, (r, hw)
        # the left halo is the s rows before the slice in the shifted
        # heads' group order, and fits the s rows in front of row 0
        assert 0 <= hl <= s and hw in (0, s)
        if hl and row0 > 0:
            assert left0 == row0 - s
        if hl and row0 == 0:
            assert boundary == oracle.WRAP and left0 == N - s


NULL = None


def call_fwd_shard(**kw):
    a = dict(N=64, row0=16, T=32, H=4, D=16, G=16, shift=8, boundary=0,
             L=64, scale=0.25, p=NULL, doc=NULL)
    a.update(kw)
    p = a["p"]
    return _lib.load().s2attn_fwd_shard(
        p, p, p, p, 1, p, a["N"], a["row0"], a["T"], a["H"], a["D"], a["G"],
        a["shift"], a["boundary"], a["L"], a["doc"], a["scale"], NULL)


def call_bwd_shard(**kw):
    a = dict(N=64, row0=16, T=32, H=4, D=16, G=16, shift=8, boundary=0,
             L=64, scale=0.25, p=NULL, doc=NULL)
    a.update(kw)
    p = a["p"]
    return _lib.load().s2attn_bwd_shard(
        p, p, p, p, 1, p, p, p, p, p, p, a["N"], a["row0"], a["T"], a["H"],
        a["D"], a["G"], a["shift"], a["boundary"], a["L"], a["doc"],
        a["scale"], NULL)


def _aligned_buffer():
    buf = (ctypes.c_char * 4096)()
    return buf, ((ctypes.addressof(buf) + 15) // 16) * 16


@pytest.mark.parametrize("call", [call_fwd_shard, call_bwd_shard])
def test_shard_rejects_bad_arguments(call):
    buf, p = _aligned_buffer()
    bad = [
        (dict(row0=8), _lib.S2A_EINVAL),            # not on a group edge
        (dict(T=24), _lib.S2A_EINVAL),              # not whole groups
        (dict(T=0), _lib.S2A_EINVAL),
        (dict(row0=-16), _lib.S2A_EINVAL),
        (dict(row0=48, T=32), _lib.S2A_EINVAL),     # past the end
        (dict(N=60, T=16), _lib.S2A_EINVAL),        # N % G
        (dict(H=3), _lib.S2A_EINVAL),
        (dict(L=0), _lib.S2A_EINVAL),
        (dict(L=65), _lib.S2A_EINVAL),
        (dict(shift=4), _lib.S2A_EINVAL),
        (dict(boundary=3), _lib.S2A_EINVAL),
        (dict(D=24), _lib.S2A_EUNSUPPORTED),
        (dict(scale=float("nan")), _lib.S2A_EINVAL),
        (dict(doc=p + 2), _lib.S2A_EINVAL),
        (dict(p=NULL), _lib.S2A_EINVAL),            # NULL tensors
        (dict(p=p + 8), _lib.S2A_EINVAL),           # misaligned tensors
    ]
    for kw, want in bad:
        kw = dict({"p": p}, **kw)
        assert call(**kw) == want, kw
        assert _lib.load().s2attn_last_error().decode() != ""


def test_shard_halo_rejects_bad_arguments():
    lib = _lib.load()
    out = [ctypes.c_int(0) for _ in range(3)]
    refs = [ctypes.byref(o) for o in out]
    assert lib.s2attn_shard_halo(64, 8, 32, 16, 8, 0, 64, *refs) \
        == _lib.S2A_EINVAL
    assert lib.s2attn_shard_halo(64, 0, 32, 16, 8, 0, 64, None, *refs[1:]) \
        == _lib.S2A_EINVAL
    assert lib.s2attn_shard_halo(64, 0, 32, 16, 8, 0, 64, *refs) \
        == _lib.S2A_OK


@pytest.mark.parametrize("boundary", BOUNDS)
@pytest.mark.parametrize("N,G,P,L", [(64, 16, 4, 64), (64, 16, 4, 50),
                                     (96, 16, 3, 90), (48, 8, 6, 7),
                                     (64, 32, 2, 40), (32, 32, 1, 30)])
def test_shard_pairs_match_oracle_enumeration(boundary, N, G, P, L):
    # the work of one slice: allowed pairs whose query lies in it, counted
    # from the oracle's adjacency rows of the slice
    T = N // P
    for half in (0, 1):
        shift = half * G // 2
        tot = [0, 0]
        for r in range(P):
            rows = np.arange(r * T, (r + 1) * T)
            want = tuple(int(oracle.adjacency_block(c, rows, N, G, shift,
                                                    boundary, L).sum())
                         for c in (0, 1))
            got = work.shard_pairs(N, r * T, T, G, shift, boundary, L)
            assert got == want, (r, got, want)
            tot = [tot[0] + got[0], tot[1] + got[1]]
        assert tuple(tot) == work.allowed_pairs(N, G, shift, boundary, L)
