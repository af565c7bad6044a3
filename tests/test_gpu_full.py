"""GPU parity at the full workload sizes, in the launch configuration the
bench times.  The GPU computes the whole tensor; the float64 oracle
recomputes sampled outputs it can produce exactly on their own:

* o, lse, dq of a query row need only that row's visible keys;
* dk, dv of a key need every query that sees it; for keys in the last R
  slots of a group those are exactly the last R slots of the group.

Samples cover one head of each class, the first, a middle and the last
group (the wrapped group under WRAP and CYCLIC, the short tail under
SPLIT), the first and last R slots of each, and for padded inputs the slots
around the valid-length boundary and wherever a group's positions jump."""
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
                   doc=None, ds=False):
    shift = G // 2
    sc = scale_for(D)
    heads = [1, H - 2]             # one head of each class
    say(f"config {config} B={B} N={N} H={H} D={D} G={G} L={L} "
        f"boundary={boundary} bwd={with_bwd} "
        f"documents={None if doc is None else int(doc.max()) + 1} "
        f"stored_ds={ds}")
    dev, host = gen(config, variant, B, N, H, D, L, heads, with_bwd)
    dd = None if doc is None else torch.from_numpy(doc).cuda()
    o, lse = s2a.fwd(dev["q"], dev["k"], dev["v"], G=G, shift=shift,
                     boundary=boundary, valid_len=L, scale=sc, doc_ids=dd)
    if with_bwd:
        dq, dk, dv = s2a.bwd(dev["q"], dev["k"], dev["v"], o, lse, dev["do"],
                             G=G, shift=shift, boundary=boundary,
                             valid_len=L, scale=sc, doc_ids=dd)
    if with_bwd and ds:
        # the stored-dS backward: dk, dv bit for bit those of the
        # recompute path, dq checked against the oracle below
        dq0, dk0, dv0 = dq, dk, dv
        dq, dk, dv = s2a.bwd_ds(dev["q"], dev["k"], dev["v"], o, lse,
                                dev["do"], G=G, shift=shift,
                                boundary=boundary, valid_len=L, scale=sc)
        torch.cuda.synchronize()
        assert torch.equal(dk, dk0) and torch.equal(dv, dv0)
        say(f"  dq vs recompute path: max|d|="
            f"{(dq - dq0).abs().max().item():.3e}")
        del dq0, dk0, dv0
    torch.cuda.synchronize()
    # padded rows are exactly zero everywhere (cheap to check in full)
    if L < N:
        assert torch.all(o[:, L:] == 0)
        assert torch.all(torch.isneginf(lse[:, :, L:]))
        if with_bwd:
            for t in (dq, dk, dv):
                assert torch.all(t[:, L:] == 0)
    errs = {n: [] for n in ("o", "lse", "dq", "dk", "dv")}
    for hi, h in enumerate(heads):
        cls = int(h >= H // 2)
        for g, (rows, tail) in sample_rows(N, G, shift, boundary, L, cls,
                                           doc).items():
            args = (host["q"], host["k"], host["v"])
            if with_bwd:
                rdq, rdk, rdv, ro, rlse = oracle.backward(
                    *args, host["do"], G, shift, boundary, L, sc, heads=[hi],
                    rows=rows, doc=doc)
            else:
                ro, rlse = oracle.forward(*args, G, shift, boundary, L, sc,
                                          heads=[hi], rows=rows, doc=doc)
            ri = torch.as_tensor(rows, device="cuda")
            ti = torch.as_tensor(tail, device="cuda")
            errs["o"].append(np.abs(o[:, ri, h].double().cpu().numpy()
                                    - ro[:, rows, hi]))
            lg = lse[:, h, ri].double().cpu().numpy()
            lw = rlse[:, hi, rows]
            fin = np.isfinite(lw)
            assert np.array_equal(fin, np.isfinite(lg))
            errs["lse"].append(np.abs(lg[fin] - lw[fin]))
            if with_bwd:
                errs["dq"].append(np.abs(dq[:, ri, h].double().cpu().numpy()
                                         - rdq[:, rows, hi]))
                errs["dk"].append(np.abs(dk[:, ti, h].double().cpu().numpy()
                                         - rdk[:, tail, hi]))
                errs["dv"].append(np.abs(dv[:, ti, h].double().cpu().numpy()
                                         - rdv[:, tail, hi]))
    for name, lst in errs.items():
        if not lst:
            continue
        e = np.concatenate([x.ravel() for x in lst])
        say(f"  {name}: {e.size} sampled values, max|d|={e.max():.3e} "
            f"mean|d|={e.mean():.3e}")
        if name == "lse":
            assert e.max() <= LSE_TOL
        else:
            assert e.max() <= ATOL_MAX and e.mean() <= ATOL_MEAN


def test_7b_layer_forward_split_8k():
    check_workload(2, 0, 1, 8192, 32, 128, 2048, syn.SPLIT, 8192, False)


def test_headline_forward_backward_wrap_32k():
    check_workload(3, 0, 1, 32768, 32, 128, 8192, syn.WRAP, 32768, True)


@pytest.mark.parametrize("G", [12288, 6144, 3072, 2048, 1536])
def test_ratio_sweep_split(G):
    check_workload(4, [12288, 6144, 3072, 2048, 1536].index(G), 2, 12288, 32,
                   128, G, syn.SPLIT, 12288, True)


def test_headline_shape_cyclic_32k():
    # the cyclic-causal boundary variant at the headline shape
    check_workload(3, 2, 1, 32768, 32, 128, 8192, syn.CYCLIC, 32768, True)


@pytest.mark.parametrize("boundary", [syn.WRAP, syn.SPLIT, syn.CYCLIC])
def test_ragged_100k(boundary):
    check_workload(5, boundary, 1, 102400, 32, 128, 25600, boundary, 100000,
                   True)


@pytest.mark.parametrize("boundary", [syn.WRAP, syn.CYCLIC])
def test_headline_stored_ds_32k(boundary):
    check_workload(3, boundary, 1, 32768, 32, 128, 8192, boundary, 32768,
                   True, ds=True)


def test_ratio_sweep_stored_ds_smallest_group():
    check_workload(4, 4, 2, 12288, 32, 128, 1536, syn.SPLIT, 12288, True,
                   ds=True)


@pytest.mark.parametrize("boundary", [syn.WRAP, syn.CYCLIC])
def test_ragged_100k_stored_ds(boundary):
    check_workload(5, boundary, 1, 102400, 32, 128, 25600, boundary, 100000,
                   True, ds=True)


@pytest.mark.parametrize("boundary", [syn.WRAP, syn.CYCLIC])
def test_headline_shape_documents_32k(boundary):
    # packed samples of mean length 1000 (as bench.py --docs 1000), the
    # headline shape, the document-masked kernels
    doc = syn.make_doc_ids(8000, 1, 32768, 1000)
    check_workload(3, 3, 1, 32768, 32, 128, 8192, boundary, 32768, True,
                   doc=doc)


@pytest.mark.parametrize("with_docs", [False, True])
def test_long_group(with_docs):
    # one group of 81,920 tokens (1,280 tiles of 64): under a document mask
    # the tiles past the 1,024 whose IDs the kernels track are all walked
    N = 81920
    doc = syn.make_doc_ids(8100, 1, N, 3000) if with_docs else None
    check_workload(6, int(with_docs), 1, N, 2, 64, N, syn.WRAP, N - 20, True,
                   doc=doc)
