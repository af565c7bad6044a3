"""GPU parity of the document mask (packed sequences) against the float64
oracle: a query reads only keys of its own document, in both head classes
and every boundary variant.  Documents are drawn with geometric lengths
(short and long samples mixed) plus forced boundaries inside a group, on an
original group boundary and on a shifted one; every output element is
compared."""
import numpy as np
import pytest
import torch

import oracle
import synthetic as syn
from gpu_helpers import (ATOL_MAX, ATOL_MEAN, LSE_TOL, compare, compare_lse,
                         say, scale_for, to_dev)

pytestmark = pytest.mark.gpu

s2a = pytest.importorskip("sparse_attention_long_attn_amd")

BNAME = {syn.WRAP: "wrap", syn.SPLIT: "split", syn.CYCLIC: "cyclic"}

# B, N, H, D, G, L, half(shift = half*G/2), mean document length
CASES = [
    (1, 64, 4, 16, 16, 64, 1, 5),
    (1, 640, 4, 32, 320, 555, 1, 90),
    (2, 768, 4, 64, 384, 700, 1, 40),
    (1, 1024, 4, 128, 256, 1000, 1, 100),
    (1, 1024, 2, 128, 256, 1024, 0, 300),
    (1, 2048, 2, 128, 512, 2000, 1, 700),
    (1, 4096, 2, 128, 1024, 3999, 1, 9),
]


def _cuts(N, G):
    s = G // 2
    return (G // 3, G, G + s, 2 * G - 1, N - s, N - s // 2)


def run_doc_case(B, N, H, D, G, L, half, mean_len, boundary, seed, relabel):
    shift = half * G // 2
    bits = syn.make_inputs(300 + seed, boundary, B, N, H, D, with_do=True, L=L)
    doc = syn.make_doc_ids(400 + seed, B, N, mean_len, cuts=_cuts(N, G))
    if relabel:  # IDs are labels only: any injective relabelling
        perm = np.random.Generator(np.random.PCG64(seed)).permutation(
            int(doc.max()) + 1).astype(np.int32)
        doc = perm[doc] * 7 - 1000
    q, k, v, do = (to_dev(bits[t]) for t in ("q", "k", "v", "do"))
    dd = torch.from_numpy(doc).cuda()
    sc = scale_for(D)
    say(f"doc case B={B} N={N} H={H} D={D} G={G} L={L} shift={shift} "
        f"{BNAME[boundary]} mean_len={mean_len} docs={int(doc.max()) + 1} "
        f"relabel={relabel}")
    o, lse = s2a.fwd(q, k, v, G=G, shift=shift, boundary=boundary,
                     valid_len=L, scale=sc, doc_ids=dd)
    dq, dk, dv = s2a.bwd(q, k, v, o, lse, do, G=G, shift=shift,
                         boundary=boundary, valid_len=L, scale=sc, doc_ids=dd)
    torch.cuda.synchronize()
    qf, kf, vf, dof = (syn.bf16_bits_to_f64(bits[t]) for t in ("q", "k", "v", "do"))
    rdq, rdk, rdv, ro, rlse = oracle.backward(qf, kf, vf, dof, G, shift,
                                              boundary, L, sc, doc=doc)
    compare("o", o.cpu().numpy(), ro, valid_rows=L)
    compare_lse(lse.cpu().numpy(), rlse, L)
    compare("dq", dq.cpu().numpy(), rdq, valid_rows=L)
    compare("dk", dk.cpu().numpy(), rdk, valid_rows=L)
    compare("dv", dv.cpu().numpy(), rdv, valid_rows=L)


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c)))
@pytest.mark.parametrize("boundary", [syn.WRAP, syn.SPLIT, syn.CYCLIC])
def test_documents_parity(case, boundary):
    i = CASES.index(case)
    run_doc_case(*case, boundary=boundary, seed=i, relabel=(i % 2 == 1))


def _run(q, k, v, do, G, boundary, L, sc, doc):
    o, lse = s2a.fwd(q, k, v, G=G, boundary=boundary, valid_len=L, scale=sc,
                     doc_ids=doc)
    dq, dk, dv = s2a.bwd(q, k, v, o, lse, do, G=G, boundary=boundary,
                         valid_len=L, scale=sc, doc_ids=doc)
    torch.cuda.synchronize()
    return o, lse, dq, dk, dv


@pytest.mark.parametrize("boundary", [syn.WRAP, syn.SPLIT, syn.CYCLIC])
def test_documents_no_leak(boundary):
    # Replacing the first document's q, k, v must leave every output of the
    # other documents unchanged.  The kernels multiply masked terms by exact
    # zeros, but a wave shares its lazy-rescale decision between rows, so a
    # changed row can move a neighbour's running max: that is an fp32
    # rounding difference (1e-6 here), where a leak would be O(1).
    B, N, H, D, G, L = 1, 2048, 4, 128, 512, 2000
    bits = syn.make_inputs(500, boundary, B, N, H, D, with_do=True, L=L)
    doc = syn.make_doc_ids(501, B, N, 200, cuts=_cuts(N, G))
    first = doc[0] == doc[0, 0]
    assert 10 < first.sum() < N - 10
    q, k, v, do = (to_dev(bits[t]) for t in ("q", "k", "v", "do"))
    dd = torch.from_numpy(doc).cuda()
    sc = scale_for(D)
    r1 = _run(q, k, v, do, G, boundary, L, sc, dd)
    sel = torch.from_numpy(first).cuda()
    g = torch.Generator(device="cuda").manual_seed(502)
    q2, k2, v2 = q.clone(), k.clone(), v.clone()
    for t in (q2, k2, v2):
        t[:, sel] = (torch.randn(t[:, sel].shape, device="cuda", generator=g)
                     * 3).to(torch.bfloat16)
    r2 = _run(q2, k2, v2, do, G, boundary, L, sc, dd)
    later = ~sel
    for name, x, y in zip(("o", "lse", "dq", "dk", "dv"), r1, r2):
        if name == "lse":
            a, b = x[..., later], y[..., later]
            fin = torch.isfinite(a)
            assert torch.equal(fin, torch.isfinite(b))
            d = (a[fin] - b[fin]).abs().max().item()
        else:
            d = (x[:, later].float() - y[:, later].float()).abs().max().item()
        say(f"  {name}: max change outside the first document {d:.3e}")
        assert d <= 1e-5, name
    # ... while the first document's own outputs did change
    assert (r1[0][:, sel] - r2[0][:, sel]).abs().max().item() > 0.1


@pytest.mark.parametrize("boundary", [syn.WRAP, syn.SPLIT, syn.CYCLIC])
def test_documents_special_cases(boundary):
    B, N, H, D, G, L = 1, 1024, 2, 128, 256, 1000
    bits = syn.make_inputs(510, boundary, B, N, H, D, with_do=True, L=L)
    q, k, v, do = (to_dev(bits[t]) for t in ("q", "k", "v", "do"))
    sc = scale_for(D)
    # one document: the numbers of no document mask, within the parity
    # bounds (the masked forward walks 64-key tiles, the unmasked one
    # 32-key tiles, so the online softmax rounds P against other running
    # maxima), and -inf in the same places
    plain = _run(q, k, v, do, G, boundary, L, sc, None)
    one = _run(q, k, v, do, G, boundary, L, sc,
               torch.zeros((B, N), dtype=torch.int32, device="cuda"))
    for name, x, y in zip(("o", "lse", "dq", "dk", "dv"), plain, one):
        fin = torch.isfinite(x)
        assert torch.equal(fin, torch.isfinite(y)), name
        d = (x[fin] - y[fin]).abs()
        say(f"  one document vs none, {name}: max|d|={d.max().item():.3e} "
            f"mean {d.mean().item():.3e}")
        if name == "lse":
            assert d.max().item() <= LSE_TOL, name
        else:
            assert d.max().item() <= ATOL_MAX and d.mean().item() <= ATOL_MEAN, name
    # one token per document: o = v, lse = scale q.k, dv = dO and no q/k
    # gradient, up to fp32 rounding (the softmax weight is exp of a
    # rounding residual, and dS = P (dO.v - dO.o) cancels to its rounding)
    own = torch.arange(N, dtype=torch.int32, device="cuda")[None, :].contiguous()
    o, lse, dq, dk, dv = _run(q, k, v, do, G, boundary, L, sc, own)
    checks = (
        ("o", (o[:, :L] - v[:, :L].float()).abs().max().item(), 1e-5),
        ("lse", (lse[..., :L] - ((q.float() * k.float()).sum(-1)
                                 .permute(0, 2, 1) * sc)[..., :L])
         .abs().max().item(), 1e-4),
        ("dq", dq[:, :L].abs().max().item(), 1e-4),
        ("dk", dk[:, :L].abs().max().item(), 1e-4),
        ("dv", (dv[:, :L] - do[:, :L].float()).abs().max().item(), 1e-5),
    )
    for name, d, tol in checks:
        say(f"  one token per document, {name}: max|d|={d:.3e}")
        assert d <= tol, name
