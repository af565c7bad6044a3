"""Float64 reference for S²-Attn forward, backward and group maps.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Plain numpy, dense,
slow, and written for a reader to check against the pages by eye.

Sources (titles of the pages; section / equation named per function):
  [LL]  PaperTrace "4.1.2 · LongLoRA: 用S²-Attn完成长上下文微调"
  [NB]  "精读笔记：LongLoRA — 长上下文大模型的高效微调", §3.2 S²-Attn

Conventions the pages leave open, fixed here (each is tested as stated):
  * heads h >= H/2 are the shifted class ([LL] §1, "半数heads平移半组";
    the slice Q[:, h_s:, :, :] with h_s = H/2);
  * the shift is s = G/2 to the left ([LL] §1, N=8 example "左移两位");
    when N/G == 1 the effective shift is 0, so G = N is full causal
    attention in both head classes;
  * WRAP = the original roll: the head and tail share the last rolled group
    and the triangular mask is applied in rolled order ([LL] §1, the
    paragraph on cyclic shifts and Figure 1, right);
  * SPLIT = strict-causal variant with a short first group [0, s) and a
    short last group [N-s, N) ([LL] §1, same paragraph; the visible-set
    formula N_1(i) with its lower bound s + G*floor((i-s)/G));
  * padding: pad first, then shift; the wrap point is the padded N; keys at
    positions >= L never enter a softmax ([LL] §1, "若N不能被G整除" and the
    paragraph on asserting H%2, G%2, N%G);
  * rows >= L: o = 0, lse = -inf, dq = 0, and they add nothing to dk, dv;
  * lse is the natural log of the sum of exp of the scaled logits.
"""
from __future__ import annotations

import numpy as np

WRAP = 0
SPLIT = 1
CYCLIC = 2


class OracleError(ValueError):
    pass


def validate(N: int, H: int, D: int, G: int, shift: int, boundary: int,
             L: int) -> None:
    """Launch-time asserts: H%2 == 0, G%2 == 0, N%G == 0 after padding
    ([LL] §1, paragraph on head count and group-length divisibility), the
    valid length inside [1, N], and only the two shifts the pages define,
    0 (plain grouping) and G/2 ([LL] §2, Table 1 rows)."""
    if N <= 0 or H <= 0 or D <= 0 or G <= 0:
        raise OracleError("sizes must be positive")
    if H % 2:
        raise OracleError("H must be even")
    if G % 2:
        raise OracleError("G must be even")
    if N % G:
        raise OracleError("padded N must be a multiple of G")
    if not (1 <= L <= N):
        raise OracleError("valid length must be in [1, N]")
    if shift not in (0, G // 2):
        raise OracleError("shift must be 0 or G/2")
    if boundary not in (WRAP, SPLIT, CYCLIC):
        raise OracleError("boundary must be WRAP, SPLIT or CYCLIC")


def effective_shift(N: int, G: int, shift: int) -> int:
    """With a single group (N == G) there is nothing to shift across: the
    group-ratio ablation of [LL] §1 treats ratio 1 as full attention."""
    return 0 if N // G == 1 else shift


def head_class(h: int, H: int) -> int:
    return 1 if h >= H // 2 else 0


# --------------------------------------------------------------------------
# Derivation A: straight from the index definitions
# --------------------------------------------------------------------------

def group_maps_a(N: int, G: int, shift: int, boundary: int):
    """gid[c][x], slot[c][x] for each original position x, and src[c][r], the
    original position held at row r of the regrouped layout, for head
    class c in {0, 1}.  int32 arrays of shape [2, N].

    Class 0 uses b(i) = floor(i/G) ([LL] §1, "把索引写开"; §2.2 mask M_h).
    Class 1 uses i' = i - G/2, b'(i) = floor(i'/G) ([LL] §1, same
    paragraph):
      WRAP : positions are rolled left by s, p = (x - s) mod N, and the
             rolled layout is cut into N/G groups; the last one is the
             wrapped group [N-s .. N-1, 0 .. s-1] ([LL] §1, N=8 example);
      SPLIT: gid = b'(x) + 1 in [0, N/G]; group 0 is the short head [0, s),
             group N/G the short tail [N-s, N); slots count from each
             group's first position (lower bound of N_1(i));
      CYCLIC: the partition floor(((x + s) mod N)/G) of the mask M_h^(s)
             ([LL] §2.2), renumbered so that the group holding both ends
             is the last one, as in WRAP; a slot is the rank of the
             position inside its group (causal order is original order).
    The map does not depend on the valid length (pad first, then shift)."""
    x = np.arange(N, dtype=np.int64)
    s = effective_shift(N, G, shift)
    gid = np.empty((2, N), np.int64)
    slot = np.empty((2, N), np.int64)
    src = np.empty((2, N), np.int64)
    gid[0], slot[0], src[0] = x // G, x % G, x
    if s == 0:
        gid[1], slot[1], src[1] = gid[0], slot[0], src[0]
    elif boundary == WRAP:
        p = np.mod(x - s, N)
        gid[1], slot[1] = p // G, p % G
        src[1] = np.mod(x + s, N)          # rolled row r holds x = r + s
    elif boundary == CYCLIC:
        M = N // G
        g = np.mod(np.mod(x + s, N) // G - 1, M)
        order = np.lexsort((x, g))         # by group, then by position
        gid[1] = g
        src[1] = x[order]
        rank = np.empty(N, np.int64)
        rank[order] = np.arange(N) - g[order] * G
        slot[1] = rank
    else:
        g = np.floor_divide(x - s, G) + 1
        start = np.maximum(0, s + (g - 1) * G)
        gid[1], slot[1], src[1] = g, x - start, x
    return gid.astype(np.int32), slot.astype(np.int32), src.astype(np.int32)


def adjacency_block(cls: int, rows: np.ndarray, N: int, G: int, shift: int,
                    boundary: int, L: int) -> np.ndarray:
    """Boolean rows A[i, j] (i in ``rows``, j in [0, N)) of the edge set
    key j -> query i for head class ``cls``.

    Class 0: floor(i/G) == floor(j/G) and j <= i ([LL] §2.2, M_h;
    §1, N_0(i) = {j : G*floor(i/G) <= j <= i}).
    Class 1 SPLIT: floor((i-s)/G) == floor((j-s)/G) and j <= i, which keeps
    the wrapped edges out ([LL] §1, N_1(i) = {j : s + G*floor((i-s)/G) <= j
    <= i}, with Python's floor for i < s).
    Class 1 WRAP: with p(x) = (x - s) mod N, floor(p(i)/G) == floor(p(j)/G)
    and p(j) <= p(i): the triangle is taken in rolled order, so queries
    0..s-1 read keys N-s..N-1 ([LL] §1, cyclic-shift paragraph).
    Class 1 CYCLIC: floor(((i+s) mod N)/G) == floor(((j+s) mod N)/G) and
    j <= i ([LL] §2.2, mask M_h^(s)).
    All: i < L and j < L (padding never enters the softmax)."""
    i = np.asarray(rows, dtype=np.int64)[:, None]
    j = np.arange(N, dtype=np.int64)[None, :]
    s = effective_shift(N, G, shift) if cls == 1 else 0
    if s == 0:
        a = (i // G == j // G) & (j <= i)
    elif boundary == SPLIT:
        a = (np.floor_divide(i - s, G) == np.floor_divide(j - s, G)) & (j <= i)
    elif boundary == CYCLIC:
        a = (np.mod(i + s, N) // G == np.mod(j + s, N) // G) & (j <= i)
    else:
        pi, pj = np.mod(i - s, N), np.mod(j - s, N)
        a = (pi // G == pj // G) & (pj <= pi)
    return a & (i < L) & (j < L)


def adjacency_dense(cls, N, G, shift, boundary, L):
    return adjacency_block(cls, np.arange(N), N, G, shift, boundary, L)


def allowed_pairs(N, G, shift, boundary, L, block=1024):
    """Number of allowed (query, key) pairs per head of class 0 and class 1,
    counted by enumerating the adjacency."""
    out = []
    for cls in (0, 1):
        tot = 0
        for r0 in range(0, N, block):
            rows = np.arange(r0, min(N, r0 + block))
            tot += int(adjacency_block(cls, rows, N, G, shift, boundary,
                                       L).sum())
        out.append(tot)
    return tuple(out)


def _heads_rows(H, N, heads, rows):
    heads = range(H) if heads is None else list(heads)
    rows = np.arange(N) if rows is None else np.unique(np.asarray(rows))
    return heads, rows


def _with_docs(am, doc, b, rb, cols):
    """Document mask: a query only reads keys of its own document, in both
    head classes ([LL] §1.1, paragraph on causal masks and sample packing:
    the same document-ID constraint for the original and the shifted
    partition).  doc: integer [B, N] or None."""
    if doc is None:
        return am
    return am & (doc[b, rb][:, None] == doc[b, cols][None, :])


def forward(q, k, v, G, shift, boundary, L, scale, heads=None, rows=None,
            block=256, doc=None):
    """Dense masked softmax attention over the derivation-A edge sets.

    For each valid query i with visible set S_i:
      z_ij = scale * q_i . k_j,   o_i = sum_j softmax_j(z_i) v_j
    ([LL] §3, the equation for o_i^s with scale 1/sqrt(D)), and
      lse_i = max_j z_ij + ln sum_j exp(z_ij - max_j z_ij)
    (the per-row log-sum-exp kept instead of probabilities, [LL] §1.1).

    q, k, v: float64 [B, N, H, D].  Returns o [B,N,H,D] and lse [B,H,N];
    rows >= L (and rows / heads not requested) hold o = 0, lse = -inf.
    doc: optional integer [B, N] document IDs (see _with_docs).
    Only the columns some row of a block can see are gathered: masked terms
    are exact zeros, so this changes no value."""
    B, N, H, D = q.shape
    validate(N, H, D, G, shift, boundary, L)
    heads, rows = _heads_rows(H, N, heads, rows)
    o = np.zeros((B, N, H, D), np.float64)
    lse = np.full((B, H, N), -np.inf, np.float64)
    for h in heads:
        cls = head_class(h, H)
        for r0 in range(0, len(rows), block):
            rb = rows[r0:r0 + block]
            a = adjacency_block(cls, rb, N, G, shift, boundary, L)
            cols = np.nonzero(a.any(axis=0))[0]
            live = a.any(axis=1)
            if cols.size == 0:
                continue
            for b in range(B):
                am = _with_docs(a[:, cols], doc, b, rb, cols)
                z = (q[b, rb, h] @ k[b, cols, h].T) * scale
                z = np.where(am, z, -np.inf)
                m = np.where(live, z.max(axis=1, initial=-np.inf), 0.0)
                e = np.where(am, np.exp(z - m[:, None]), 0.0)
                lsum = e.sum(axis=1)
                ob = (e @ v[b, cols, h]) / np.where(live, lsum, 1.0)[:, None]
                o[b, rb, h] = np.where(live[:, None], ob, 0.0)
                lse[b, h, rb] = np.where(live, m + np.log(
                    np.where(live, lsum, 1.0)), -np.inf)
    return o, lse


def backward(q, k, v, do, G, shift, boundary, L, scale, heads=None,
             rows=None, block=256, doc=None):
    """Gradients of sum(dO * O) with respect to q, k, v, evaluated from the
    definition.  With a_ij = exp(z_ij - lse_i) and g = dO_i, the gradient
    with respect to a logit is dL/dz_ij = a_ij * g.(v_j - o_i)
    ([LL] §3, "梯度为何也会改变"); then
      dq_i = scale * sum_j dz_ij k_j,  dk_j = scale * sum_i dz_ij q_i,
      dv_j = sum_i a_ij dO_i.
    Only in-group edges carry gradient ([LL] §1.1, "反向传播确实保持稀疏").

    Returns (dq, dk, dv, o, lse), float64.  If ``rows`` is given, only those
    queries contribute: dk/dv are then complete exactly for keys whose every
    viewer is in ``rows``."""
    B, N, H, D = q.shape
    validate(N, H, D, G, shift, boundary, L)
    heads, rows = _heads_rows(H, N, heads, rows)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    o = np.zeros((B, N, H, D), np.float64)
    lse = np.full((B, H, N), -np.inf, np.float64)
    for h in heads:
        cls = head_class(h, H)
        for r0 in range(0, len(rows), block):
            rb = rows[r0:r0 + block]
            a_ = adjacency_block(cls, rb, N, G, shift, boundary, L)
            cols = np.nonzero(a_.any(axis=0))[0]
            live = a_.any(axis=1)
            if cols.size == 0:
                continue
            for b in range(B):
                am = _with_docs(a_[:, cols], doc, b, rb, cols)
                z = (q[b, rb, h] @ k[b, cols, h].T) * scale
                z = np.where(am, z, -np.inf)
                m = np.where(live, z.max(axis=1, initial=-np.inf), 0.0)
                e = np.where(am, np.exp(z - m[:, None]), 0.0)
                lsum = np.where(live, e.sum(axis=1), 1.0)
                lse_b = m + np.log(lsum)
                a = np.where(am, np.exp(z - lse_b[:, None]), 0.0)
                ob = a @ v[b, cols, h]
                g = do[b, rb, h]
                # g.(v_j - o_i) = g.v_j - g.o_i
                gv = g @ v[b, cols, h].T
                go = np.sum(g * ob, axis=1)
                dz = a * (gv - go[:, None])
                dq[b, rb, h] = scale * (dz @ k[b, cols, h])
                dk[b, cols, h] += scale * (dz.T @ q[b, rb, h])
                dv[b, cols, h] += a.T @ g
                o[b, rb, h] = np.where(live[:, None], ob, 0.0)
                lse[b, h, rb] = np.where(live, lse_b, -np.inf)
    return dq, dk, dv, o, lse


# --------------------------------------------------------------------------
# Derivation B: shift -> regroup -> per-group causal attention -> unshift
# --------------------------------------------------------------------------

def segments(N: int, G: int, shift: int, boundary: int):
    """The groups of each head class as lists of original positions, in
    group order, obtained the way the reference implementations lay the
    tensor out ([LL] §1, "Reshape如何复用普通kernel" and the paragraph on
    forward_flashattn / forward_noflashattn):
      class 0            : arange(N) cut into N/G rows of G;
      class 1, WRAP      : np.roll(arange(N), -s) cut into N/G rows of G;
      class 1, SPLIT     : arange(N) split at s, s+G, ..., N-s;
      class 1, CYCLIC    : the rows of WRAP, each sorted by position (causal
                           order on original positions, [LL] §2.2)."""
    s = effective_shift(N, G, shift)
    M = N // G
    pos = np.arange(N, dtype=np.int64)
    c0 = list(pos.reshape(M, G))
    if s == 0:
        c1 = [seg.copy() for seg in c0]
    elif boundary == WRAP:
        c1 = list(np.roll(pos, -s).reshape(M, G))
    elif boundary == CYCLIC:
        c1 = [np.sort(row) for row in np.roll(pos, -s).reshape(M, G)]
    else:
        cuts = [s + t * G for t in range(M)]
        c1 = np.split(pos, cuts)
    return [c0, c1]


def group_maps_b(N: int, G: int, shift: int, boundary: int):
    """gid/slot/src read off the segment structure of ``segments``."""
    segs = segments(N, G, shift, boundary)
    gid = np.empty((2, N), np.int32)
    slot = np.empty((2, N), np.int32)
    src = np.empty((2, N), np.int32)
    for c in (0, 1):
        for g, seg in enumerate(segs[c]):
            gid[c, seg] = g
            slot[c, seg] = np.arange(len(seg))
        src[c] = np.concatenate(segs[c])
    return gid, slot, src


def _segment_softmax(qs, ks, pos, L, scale, dseg=None):
    n = len(pos)
    live = pos < L
    allow = np.tril(np.ones((n, n), bool)) & live[None, :] & live[:, None]
    if dseg is not None:
        allow &= dseg[:, None] == dseg[None, :]
    s = (qs @ ks.T) * scale
    s = np.where(allow, s, -np.inf)
    mx = np.where(live, s.max(axis=1, initial=-np.inf), 0.0)
    e = np.where(allow, np.exp(s - mx[:, None]), 0.0)
    tot = np.where(live, e.sum(axis=1), 1.0)
    p = e / tot[:, None]
    lse = np.where(live, mx + np.log(tot), -np.inf)
    return p, lse, live


def forward_segments(q, k, v, G, shift, boundary, L, scale, doc=None):
    """Derivation B of the forward: for every head and group, gather the
    group's rows in group order, run ordinary causal softmax attention on
    that short sequence (keys at positions >= L masked), and scatter the
    result back to the original positions (the inverse shift)."""
    B, N, H, D = q.shape
    validate(N, H, D, G, shift, boundary, L)
    segs = segments(N, G, shift, boundary)
    o = np.zeros((B, N, H, D))
    lse = np.full((B, H, N), -np.inf)
    for b in range(B):
        for h in range(H):
            for pos in segs[head_class(h, H)]:
                p, ls, live = _segment_softmax(
                    q[b, pos, h], k[b, pos, h], pos, L, scale,
                    None if doc is None else doc[b, pos])
                o[b, pos, h] = np.where(live[:, None], p @ v[b, pos, h], 0.0)
                lse[b, h, pos] = ls
    return o, lse


def backward_segments(q, k, v, do, G, shift, boundary, L, scale, doc=None):
    """Derivation B of the backward: per group, the textbook softmax
    backward dS = P * (dP - rowsum(P * dP)) with dP = dO V^T, then
    dQ = scale dS K, dK = scale dS^T Q, dV = P^T dO, scattered back."""
    B, N, H, D = q.shape
    validate(N, H, D, G, shift, boundary, L)
    segs = segments(N, G, shift, boundary)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(H):
            for pos in segs[head_class(h, H)]:
                qs, ks, vs = q[b, pos, h], k[b, pos, h], v[b, pos, h]
                p, _, live = _segment_softmax(
                    qs, ks, pos, L, scale, None if doc is None else doc[b, pos])
                g = np.where(live[:, None], do[b, pos, h], 0.0)
                dp = g @ vs.T
                ds = p * (dp - np.sum(p * dp, axis=1, keepdims=True))
                dq[b, pos, h] += scale * ds @ ks
                dk[b, pos, h] += scale * ds.T @ qs
                dv[b, pos, h] += p.T @ g
    return dq, dk, dv
