"""GPU parity at the full workload sizes, in the launch configuration the
bench times.  The GPU computes the whole tensor; the float64 oracle
recomputes the outputs it can produce exactly on their own:

* o, lse, dq of a query row need only that row's visible keys;
* dk, dv of a key need every query that sees it.  Those all lie in the
  key's own group, so running the oracle over every row of one whole group
  makes dk, dv exact for every key of that group; for keys in the last R
  slots of a group the last R slots of the group suffice.

Per workload, one head of each class is compared: every row and every key
of one whole group (the middle group in the unshifted class; the wrapped
group under WRAP and CYCLIC, a full-length group under SPLIT in the shifted
one), and sampled rows of the first, a middle and the last group (both ends
of each, the valid-length boundary, wherever a group's positions jump, the
first document starts).  A whole group of G keys is the longest walk a
dK/dV workgroup makes, G/64 query tiles.  Padded rows are checked exactly
in full.  Where the stored-dS backward supports the shape (D 64/128, no
document mask) it runs as well: its dk, dv must equal the recompute
backward's bit for bit and its dq is compared with the oracle."""
import numpy as np
import pytest
import torch

import oracle
import synthetic as syn
from gpu_helpers import ATOL_MAX, ATOL_MEAN, LSE_TOL, say, scale_for

pytestmark = pytest.mark.gpu

s2a = pytest.importorskip("sparse_attention_long_attn_amd")

R = 192   # rows per sampled slot window


def upload(bits):
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()


def gen(config, variant, B, N, H, D, L, heads, with_do):
    """Device tensors of the full inputs and float64 host copies of the
    sampled heads."""
    dev, host = {}, {}
    names = ("q", "k", "v", "do") if with_do else ("q", "k", "v")
    for t in names:
        bits = syn.normal_bf16_bits(syn.seed_for(config, variant, t),
                                    (B, N, H, D))
        if t == "do" and L < N:
            bits[:, L:] = 0
        dev[t] = upload(bits)
        host[t] = syn.bf16_bits_to_f64(bits[:, :, heads, :])
        del bits
    return dev, host


def whole_group(segs, cls, boundary, shift):
    """Index of the group compared in full for head class ``cls``."""
    if cls == 1 and shift and boundary != syn.SPLIT:
        return len(segs) - 1          # the wrapped group
    return len(segs) // 2             # a full-length middle group


def sample_rows(N, G, shift, boundary, L, cls, doc=None):
    """{group index: (query positions, tail positions)} for the groups
    sampled in head class ``cls`` (with document IDs, also around the first
    document starts inside each sampled group)."""
    segs = oracle.segments(N, G, shift, boundary)[cls]
    picks = sorted({0, len(segs) // 2, len(segs) - 1})
    out = {}
    s = oracle.effective_shift(N, G, shift)
    for g in picks:
        seg = np.asarray(segs[g])
        n = len(seg)
        slots = set(range(min(R, n))) | set(range(max(0, n - R), n))
        # around the wrap point and the valid-length boundary
        for j in range(n):
            if (j > 0 and seg[j] != seg[j - 1] + 1) or (seg[j] == L):
                slots |= set(range(max(0, j - R // 2), min(n, j + R // 2)))
        if s and cls == 1 and boundary != syn.SPLIT and g == len(segs) - 1:
            slots |= set(range(max(0, s - R // 2), min(n, s + R // 2)))
        if doc is not None:
            starts = [j for j in range(1, n) if doc[0, seg[j]] != doc[0, seg[j - 1]]]
            for j in starts[:4]:
                slots |= set(range(max(0, j - R // 4), min(n, j + R // 4)))
        rows = seg[sorted(slots)]
        tail = seg[max(0, n - R):]
        out[g] = (rows, tail)
    return out


def check_workload(config, variant, B, N, H, D, G, boundary, L, with_bwd,
                   doc=None, ds=None, full=True, key_range=None):
    """``full``: compare one whole group per head class (every row and
    every key); ``key_range``: (positions of keys, rows that are all their
    viewers) compared in addition, for the shifted-class head."""
    shift = G // 2
    sc = scale_for(D)
    heads = [1, H - 2]             # one head of each class
    if ds is None:
        ds = with_bwd and doc is None and D in (64, 128)
    say(f"config {config} B={B} N={N} H={H} D={D} G={G} L={L} "
        f"boundary={boundary} bwd={with_bwd} "
        f"documents={None if doc is None else int(doc.max()) + 1} "
        f"stored_ds={ds} whole_group={full}")
    dev, host = gen(config, variant, B, N, H, D, L, heads, with_bwd)
    dd = None if doc is None else torch.from_numpy(doc).cuda()
    o, lse = s2a.fwd(dev["q"], dev["k"], dev["v"], G=G, shift=shift,
                     boundary=boundary, valid_len=L, scale=sc, doc_ids=dd)
    dqs = {}
    if with_bwd:
        dq, dk, dv = s2a.bwd(dev["q"], dev["k"], dev["v"], o, lse, dev["do"],
                             G=G, shift=shift, boundary=boundary,
                             valid_len=L, scale=sc, doc_ids=dd)
        dqs["recompute"] = dq
    if with_bwd and ds:
        # the stored-dS backward: dk, dv bit for bit those of the
        # recompute path, dq checked against the oracle below
        dq2, dk2, dv2 = s2a.bwd_ds(dev["q"], dev["k"], dev["v"], o, lse,
                                   dev["do"], G=G, shift=shift,
                                   boundary=boundary, valid_len=L, scale=sc)
        torch.cuda.synchronize()
        assert torch.equal(dk, dk2) and torch.equal(dv, dv2)
        say(f"  dq stored dS vs recompute: max|d|="
            f"{(dq2 - dq).abs().max().item():.3e}")
        dqs["stored dS"] = dq2
        del dk2, dv2
    torch.cuda.synchronize()
    # padded rows are exactly zero everywhere (cheap to check in full)
    if L < N:
        assert torch.all(o[:, L:] == 0)
        assert torch.all(torch.isneginf(lse[:, :, L:]))
        if with_bwd:
            for t in (*dqs.values(), dk, dv):
                assert torch.all(t[:, L:] == 0)
    errs = {}

    def add(name, got, want):
        errs.setdefault(name, []).append(np.abs(got - want))

    def cmp_rows(h, hi, rows, ro, rlse, rdq):
        ri = torch.as_tensor(rows, device="cuda")
        add("o", o[:, ri, h].double().cpu().numpy(), ro[:, rows, hi])
        lg = lse[:, h, ri].double().cpu().numpy()
        lw = rlse[:, hi, rows]
        fin = np.isfinite(lw)
        assert np.array_equal(fin, np.isfinite(lg))
        add("lse", lg[fin], lw[fin])
        for name, t in dqs.items():
            add(f"dq ({name})", t[:, ri, h].double().cpu().numpy(),
                rdq[:, rows, hi])

    def cmp_keys(h, hi, keys, rdk, rdv, tag):
        ki = torch.as_tensor(keys, device="cuda")
        add(f"dk ({tag})", dk[:, ki, h].double().cpu().numpy(),
            rdk[:, keys, hi])
        add(f"dv ({tag})", dv[:, ki, h].double().cpu().numpy(),
            rdv[:, keys, hi])

    def run_oracle(hi, rows):
        args = (host["q"], host["k"], host["v"])
        if with_bwd:
            return oracle.backward(*args, host["do"], G, shift, boundary, L,
                                   sc, heads=[hi], rows=rows, doc=doc)
        ro, rlse = oracle.forward(*args, G, shift, boundary, L, sc,
                                  heads=[hi], rows=rows, doc=doc)
        return None, None, None, ro, rlse

    for hi, h in enumerate(heads):
        cls = int(h >= H // 2)
        segs = oracle.segments(N, G, shift, boundary)[cls]
        if full:
            gw = whole_group(segs, cls, boundary, shift)
            rows = np.asarray(segs[gw])
            say(f"  head {h}: whole group {gw} ({len(rows)} rows)")
            rdq, rdk, rdv, ro, rlse = run_oracle(hi, rows)
            cmp_rows(h, hi, rows, ro, rlse, rdq)
            if with_bwd:
                cmp_keys(h, hi, rows, rdk, rdv, "whole group")
        for g, (rows, tail) in sample_rows(N, G, shift, boundary, L, cls,
                                           doc).items():
            rdq, rdk, rdv, ro, rlse = run_oracle(hi, rows)
            cmp_rows(h, hi, rows, ro, rlse, rdq)
            if with_bwd:
                cmp_keys(h, hi, tail, rdk, rdv, "group tails")
        if key_range is not None and with_bwd and cls == 1:
            keys, rows = key_range
            say(f"  head {h}: keys {keys[0]}..{keys[-1]} from "
                f"{len(rows)} rows")
            rdq, rdk, rdv, ro, rlse = run_oracle(hi, rows)
            cmp_keys(h, hi, keys, rdk, rdv, "key range")
    for name, lst in errs.items():
        e = np.concatenate([x.ravel() for x in lst])
        say(f"  {name}: {e.size} values, max|d|={e.max():.3e} "
            f"mean|d|={e.mean():.3e}")
        if name == "lse":
            assert e.max() <= LSE_TOL
        else:
            assert e.max() <= ATOL_MAX and e.mean() <= ATOL_MEAN


def test_7b_layer_forward_split_8k():
    check_workload(2, 0, 1, 8192, 32, 128, 2048, syn.SPLIT, 8192, False)


@pytest.mark.parametrize("boundary", [syn.WRAP, syn.SPLIT, syn.CYCLIC])
def test_headline_shape_32k(boundary):
    # the headline workload (WRAP, the one the bench times) and the other
    # two boundary variants at its shape; both backwards
    check_workload(3, boundary, 1, 32768, 32, 128, 8192, boundary, 32768,
                   True)


@pytest.mark.parametrize("G", [12288, 6144, 3072, 2048, 1536])
def test_ratio_sweep_split(G):
    check_workload(4, [12288, 6144, 3072, 2048, 1536].index(G), 2, 12288, 32,
                   128, G, syn.SPLIT, 12288, True)


@pytest.mark.parametrize("boundary", [syn.WRAP, syn.SPLIT, syn.CYCLIC])
def test_ragged_100k(boundary):
    check_workload(5, boundary, 1, 102400, 32, 128, 25600, boundary, 100000,
                   True)


@pytest.mark.parametrize("boundary", [syn.WRAP, syn.CYCLIC])
def test_headline_shape_documents_32k(boundary):
    # packed samples of mean length 1000 (as bench.py --docs 1000), the
    # headline shape, the document-masked kernels
    doc = syn.make_doc_ids(8000, 1, 32768, 1000)
    check_workload(3, 3, 1, 32768, 32, 128, 8192, boundary, 32768, True,
                   doc=doc)


@pytest.mark.parametrize("with_docs", [False, True])
def test_long_group(with_docs):
    # One group of 81,920 tokens (1,280 tiles of 64).  Under a document
    # mask a workgroup tracks the IDs of the first 1,024 tiles of its walk
    # and walks every tile past them; the key blocks whose walks reach past
    # that are the first 16,384 keys, compared here in full (their viewers
    # are the queries of their own documents).
    N, L = 81920, 81920 - 20
    doc = syn.make_doc_ids(8100, 1, N, 3000) if with_docs else None
    key_range = None
    if with_docs:
        keys = np.arange(16384)
        last = int(np.nonzero(doc[0] == doc[0, keys[-1]])[0].max())
        key_range = (keys, np.arange(min(L, last + 1)))
    check_workload(6, int(with_docs), 1, N, 2, 64, N, syn.WRAP, L, True,
                   doc=doc, full=False, key_range=key_range)
