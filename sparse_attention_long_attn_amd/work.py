"""Host-side work accounting: allowed pairs, useful FLOPs, algorithmic bytes.

Pair counts are the closed forms of the edge sets (PaperTrace "4.1.2 ·
LongLoRA: 用S²-Attn完成长上下文微调", §1, complexity paragraph: a group of
length n holds n(n+1)/2 causal pairs, so a class of M full groups holds
M*G*(G+1)/2 ~ NG/2).  With a valid length L < N, a group's pairs are those
among its valid members in group order.  Useful FLOPs count 4*D per allowed
pair for the forward (2D for QK^T, 2D for PV) and 10*D for the backward.
"""
from __future__ import annotations

WRAP, SPLIT, CYCLIC = 0, 1, 2


def _groups(N, G, shift, boundary, cls):
    """Each group of a head class as its runs of consecutive positions,
    [(first, end), ...] in group (causal) order."""
    M = N // G
    s = 0 if M == 1 else shift
    if cls == 0 or s == 0:
        return [[(g * G, g * G + G)] for g in range(M)]
    if boundary == SPLIT:
        return ([[(0, s)]] + [[(s + g * G, s + g * G + G)] for g in range(M - 1)]
                + [[(N - s, N)]])
    inner = [[(g * G + s, g * G + s + G)] for g in range(M - 1)]
    if boundary == WRAP:                 # rolled order: N-s..N-1, 0..s-1
        return inner + [[(N - s, N), (0, s)]]
    return inner + [[(0, s), (N - s, N)]]  # CYCLIC: position order


def _pairs_in_group(runs, L):
    """Causal pairs among the valid members of a group given as runs."""
    # pairs = sum over valid slots j of (number of valid slots <= j)
    tot = 0
    cnt = 0
    for a, b in runs:
        v = max(0, min(b, L) - a)      # valid positions of the run
        tot += v * cnt + v * (v + 1) // 2
        cnt += v
    return tot


def allowed_pairs(N, G, shift, boundary, L):
    """Allowed (query, key) pairs per head of class 0 and class 1."""
    out = []
    for cls in (0, 1):
        out.append(sum(_pairs_in_group(runs, L)
                       for runs in _groups(N, G, shift, boundary, cls)))
    return tuple(out)


def shard_pairs(N, row0, T, G, shift, boundary, L):
    """Allowed pairs per head of class 0 and class 1 whose query lies in
    the slice [row0, row0 + T): the work of that slice under sequence
    parallelism (its keys may lie outside it).  A valid query at slot j of
    a group reads the valid slots up to j."""
    out = []
    hi_q = min(L, row0 + T)
    for cls in (0, 1):
        tot = 0
        for runs in _groups(N, G, shift, boundary, cls):
            cnt = 0  # valid slots before the current run
            for a, b in runs:
                lo, hi = max(a, row0), min(b, hi_q)
                if hi > lo:  # queries x in [lo, hi) read cnt + x - a + 1 keys
                    n = hi - lo
                    tot += n * (cnt - a + 1) + (lo + hi - 1) * n // 2
                cnt += max(0, min(b, L) - a)
        out.append(tot)
    return tuple(out)


def total_pairs(B, N, H, G, shift, boundary, L):
    c0, c1 = allowed_pairs(N, G, shift, boundary, L)
    return B * (H // 2) * (c0 + c1)


def useful_flops(B, N, H, D, G, shift, boundary, L):
    """(forward, backward) useful FLOPs: 4*D and 10*D per allowed pair."""
    p = total_pairs(B, N, H, G, shift, boundary, L)
    return 4 * D * p, 10 * D * p


def algorithmic_bytes(B, N, H, D, o_bytes=4):
    """(forward, backward) minimum HBM bytes of one pass.

    forward : read q, k, v (bf16); write o and lse
    backward: read q, k, v, dout (bf16), o, lse; write delta then read it;
              write dq, dk, dv (fp32)"""
    e = B * N * H * D
    rows = B * H * N
    fwd = 3 * 2 * e + o_bytes * e + 4 * rows
    bwd = 4 * 2 * e + o_bytes * e + 3 * 4 * e + 3 * 4 * rows
    return fwd, bwd


def doc_pairs(N, G, shift, boundary, L, doc_row):
    """Allowed pairs per head of class 0 and class 1 under a document mask
    (one batch row's int [N] document IDs): inside a group a valid query
    reads every earlier-or-equal valid slot with its own ID, so a label that
    occurs n times among a group's valid members contributes n(n+1)/2."""
    import numpy as np
    doc_row = np.asarray(doc_row)
    out = []
    for cls in (0, 1):
        tot = 0
        for runs in _groups(N, G, shift, boundary, cls):
            ids = np.concatenate([doc_row[a:min(b, L)] for a, b in runs
                                  if min(b, L) > a] or [np.zeros(0, int)])
            if ids.size:
                _, n = np.unique(ids, return_counts=True)
                tot += int(np.sum(n * (n + 1) // 2))
        out.append(tot)
    return tuple(out)


def total_doc_pairs(B, N, H, G, shift, boundary, L, doc):
    """Allowed pairs of the whole batch under document IDs doc [B, N]."""
    tot = 0
    for b in range(B):
        c0, c1 = doc_pairs(N, G, shift, boundary, L, doc[b])
        tot += (H // 2) * (c0 + c1)
    return tot
