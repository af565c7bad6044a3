"""GPU parity of the sequence-parallel shard calls.  One GPU plays every
rank in turn: the sequence is cut into P slices on group edges, each
slice's halo (the rows s2attn_shard_halo names) is copied in front of its
K/V as a neighbour's send would deliver it, the slice runs fwd_shard and
bwd_shard, and the halo rows' partial dK/dV are added to their owners'
rows.  The assembled outputs are compared with the float64 oracle over the
whole sequence, element by element, and with the unsharded kernels: bit
for bit wherever the slice numbers its groups' slots as the whole sequence
does and no partial sum is involved ([LL] §1.1, the paragraphs on
sequence-parallel communication)."""
import numpy as np
import pytest
import torch

import oracle
import synthetic as syn
from gpu_helpers import compare, compare_lse, say, scale_for, to_dev

pytestmark = pytest.mark.gpu

s2a = pytest.importorskip("sparse_attention_long_attn_amd")

BNAME = {syn.WRAP: "wrap", syn.SPLIT: "split", syn.CYCLIC: "cyclic"}


def run_shards(q, k, v, do, N, G, shift, boundary, L, P, doc=None,
               out_dtype=torch.float32):
    """q, k, v, do [N, H, D] bf16 (one sequence), doc [N] int32 or None.
    Returns the assembled (o, lse, dq, dk, dv), the halo of each slice and
    the rows that received another slice's partials."""
    _, H, D = q.shape
    T = N // P
    s = shift if N // G > 1 else 0
    R = 2 * s  # room for the left halo and, under CYCLIC, the wrap halo
    dev = q.device
    o_all = torch.zeros((N, H, D), dtype=out_dtype, device=dev)
    lse_all = torch.empty((H, N), dtype=torch.float32, device=dev)
    dq_all = torch.zeros((N, H, D), dtype=torch.float32, device=dev)
    dk_all = torch.zeros((N, H, D), dtype=torch.float32, device=dev)
    dv_all = torch.zeros((N, H, D), dtype=torch.float32, device=dev)
    halos, partial_rows = [], set()
    kw = dict(N=N, G=G, shift=shift, boundary=boundary, valid_len=L)
    for r in range(P):
        row0 = r * T
        left0, hl, hw = s2a.shard_halo(N, row0, T, G=G, shift=shift,
                                       boundary=boundary, valid_len=L)
        halos.append((left0, hl, hw))
        sl = slice(row0, row0 + T)

        def ext(x):  # the slice's rows behind R halo rows
            # the halo rows a slice does not read hold finite filler
            e = torch.zeros((R + T,) + tuple(x.shape[1:]), dtype=x.dtype,
                            device=dev)
            e[R:] = x[sl]
            if hl:
                e[R - hl:R] = x[left0:left0 + hl]
            if hw:
                e[R - 2 * s:R - 2 * s + hw] = x[0:hw]
            return e

        kx, vx = ext(k), ext(v)
        dx = None if doc is None else ext(doc)
        o, lse = s2a.fwd_shard(q[sl], kx, vx, row0=row0, out_dtype=out_dtype,
                               doc_ext=dx, **kw)
        dq, dkx, dvx = s2a.bwd_shard(q[sl], kx, vx, o, lse, do[sl],
                                     row0=row0, doc_ext=dx, **kw)
        o_all[sl], lse_all[:, sl], dq_all[sl] = o, lse, dq
        dk_all[sl] += dkx[R:]
        dv_all[sl] += dvx[R:]
        # partial gradients of the halo keys go back to their owners
        if hl:
            dk_all[left0:left0 + hl] += dkx[R - hl:R]
            dv_all[left0:left0 + hl] += dvx[R - hl:R]
            partial_rows.update(range(left0, left0 + hl))
        if hw:
            dk_all[0:hw] += dkx[R - 2 * s:R - 2 * s + hw]
            dv_all[0:hw] += dvx[R - 2 * s:R - 2 * s + hw]
            partial_rows.update(range(hw))
    torch.cuda.synchronize()
    return (o_all, lse_all, dq_all, dk_all, dv_all), halos, partial_rows


# N, H, D, G, L, P, shift = half * G/2, mean document length (0: none)
CASES = [
    (1024, 4, 128, 256, 1024, 2, 1, 0),
    (1024, 4, 128, 256, 947, 4, 1, 0),    # first slice's WRAP halo padded
    (1024, 4, 128, 256, 830, 4, 1, 0),    # the last slice mostly padding
    (1024, 4, 128, 256, 1000, 1, 1, 0),   # one slice: halos are its own rows
    (768, 4, 64, 256, 700, 3, 1, 0),
    (512, 4, 32, 64, 500, 4, 1, 0),
    (256, 4, 16, 32, 251, 8, 1, 0),       # halos of 16 rows, mixed waves
    (1024, 4, 128, 256, 1000, 4, 0, 0),   # no shift: no halo at all
    (1024, 4, 128, 256, 1000, 4, 1, 90),  # document mask
    (768, 4, 64, 256, 768, 3, 1, 30),
]


def _inputs(i, boundary, N, H, D, L, mean_len, G):
    bits = syn.make_inputs(900 + i, boundary, 1, N, H, D, with_do=True, L=L)
    doc = None
    if mean_len:
        doc = syn.make_doc_ids(910 + i, 1, N, mean_len,
                               cuts=(G // 3, G, G + G // 2))
    return bits, doc


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c)))
@pytest.mark.parametrize("boundary", [syn.WRAP, syn.SPLIT, syn.CYCLIC])
def test_shards_match_oracle_and_whole_sequence(case, boundary):
    N, H, D, G, L, P, half, mean_len = case
    i = CASES.index(case)
    shift = half * G // 2
    s = shift if N // G > 1 else 0
    bits, doc = _inputs(i, boundary, N, H, D, L, mean_len, G)
    say(f"shards N={N} H={H} D={D} G={G} L={L} P={P} shift={shift} "
        f"{BNAME[boundary]} docs={0 if doc is None else int(doc.max()) + 1}")
    q, k, v, do = (to_dev(bits[t])[0] for t in ("q", "k", "v", "do"))
    dd = None if doc is None else torch.from_numpy(doc[0]).cuda()
    sc = scale_for(D)
    (o, lse, dq, dk, dv), halos, prow = run_shards(q, k, v, do, N, G, shift,
                                                   boundary, L, P, doc=dd)
    say(f"  halos (left first, left rows, wrap rows): {halos}")

    # against the float64 oracle over the whole sequence
    qf, kf, vf, dof = (syn.bf16_bits_to_f64(bits[t])
                       for t in ("q", "k", "v", "do"))
    rdq, rdk, rdv, ro, rlse = oracle.backward(qf, kf, vf, dof, G, shift,
                                              boundary, L, sc, doc=doc)
    compare("o", o.cpu().numpy()[None], ro, valid_rows=L)
    compare_lse(lse.cpu().numpy()[None], rlse, L)
    compare("dq", dq.cpu().numpy()[None], rdq, valid_rows=L)
    compare("dk", dk.cpu().numpy()[None], rdk, valid_rows=L)
    compare("dv", dv.cpu().numpy()[None], rdv, valid_rows=L)

    # against the unsharded kernels
    kw = dict(G=G, shift=shift, boundary=boundary, valid_len=L, scale=sc,
              doc_ids=None if dd is None else dd[None].contiguous())
    go, glse = s2a.fwd(q[None], k[None], v[None], **kw)
    gdq, gdk, gdv = s2a.bwd(q[None], k[None], v[None], go, glse, do[None],
                            **kw)
    torch.cuda.synchronize()
    go, glse, gdq, gdk, gdv = go[0], glse[0], gdq[0], gdk[0], gdv[0]
    # The slices number slots as the whole sequence does when the first
    # slice's WRAP halo is whole (else its first group starts later), and
    # waves of 32 rows then never mix halo and slice rows when s % 32 == 0.
    same_slots = s % 32 == 0 and halos[0][1] in (0, s) and \
        not (boundary == syn.WRAP and s and halos[0][1] < s)
    own = torch.ones(N, dtype=torch.bool, device="cuda")
    own[list(prow)] = False
    for name, a, b in (("o", o, go), ("dq", dq, gdq)):
        d = (a - b).abs().max().item()
        say(f"  {name} vs unsharded: max|d|={d:.3e}")
        if same_slots:
            assert torch.equal(a, b), name
    fin = torch.isfinite(glse)
    assert torch.equal(fin, torch.isfinite(lse))
    if same_slots:
        assert torch.equal(lse, glse)
    for name, a, b in (("dk", dk, gdk), ("dv", dv, gdv)):
        d_own = (a[own] - b[own]).abs().max().item() if own.any() else 0.0
        d_par = (a[~own] - b[~own]).abs().max().item() if (~own).any() else 0.0
        say(f"  {name} vs unsharded: own rows max|d|={d_own:.3e}, rows with "
            f"halo partials max|d|={d_par:.3e}")
        if same_slots:
            assert torch.equal(a[own], b[own]), name
            # a partial sum reorders fp32 additions only
            assert d_par <= 1e-4, name
        # (otherwise both runs are within the oracle bound, checked above)


def test_shards_with_bf16_output():
    N, H, D, G, L, P = 1024, 4, 128, 256, 1024, 4
    bits, _ = _inputs(50, syn.WRAP, N, H, D, L, 0, G)
    q, k, v, do = (to_dev(bits[t])[0] for t in ("q", "k", "v", "do"))
    (o, lse, dq, dk, dv), _, _ = run_shards(
        q, k, v, do, N, G, G // 2, syn.WRAP, L, P, out_dtype=torch.bfloat16)
    go, glse = s2a.fwd(q[None], k[None], v[None], G=G, valid_len=L,
                       out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(o, go[0]) and torch.equal(lse, glse[0])


@pytest.mark.parametrize("boundary", [syn.WRAP, syn.SPLIT, syn.CYCLIC])
def test_headline_shape_in_four_slices(boundary):
    # B=1 N=32768 H=32 D=128 G=8192 in four slices of 8192 rows (one group
    # each, as on four devices): the slices' outputs equal the unsharded
    # kernels' bit for bit, except the halo rows' partial sums.
    N, H, D, G, P = 32768, 32, 128, 8192, 4
    L = N - 300
    s = G // 2
    g = torch.Generator(device="cuda").manual_seed(77 + boundary)
    q, k, v, do = (torch.randn((N, H, D), device="cuda", generator=g)
                   .to(torch.bfloat16) for _ in range(4))
    do[L:] = 0
    say(f"headline shape in {P} slices, {BNAME[boundary]}, L={L}")
    (o, lse, dq, dk, dv), halos, prow = run_shards(q, k, v, do, N, G, s,
                                                   boundary, L, P)
    say(f"  halos: {halos}")
    kw = dict(G=G, boundary=boundary, valid_len=L)
    go, glse = s2a.fwd(q[None], k[None], v[None], **kw)
    gdq, gdk, gdv = s2a.bwd(q[None], k[None], v[None], go, glse, do[None],
                            **kw)
    torch.cuda.synchronize()
    go, glse, gdq, gdk, gdv = go[0], glse[0], gdq[0], gdk[0], gdv[0]
    first_whole = halos[0][1] in (0, s)
    # under WRAP the padded tail shortens the first slice's halo, so its
    # first shifted group numbers slots differently: compare those rows
    # (the shifted heads' rows 0..s-1) within rounding
    rows = torch.ones(N, dtype=torch.bool, device="cuda")
    if not first_whole:
        rows[:s] = False
    for name, a, b in (("o", o, go), ("dq", dq, gdq)):
        assert torch.equal(a[rows], b[rows]), name
        d = (a[~rows] - b[~rows]).abs().max().item() if (~rows).any() else 0
        say(f"  {name}: bitwise on {int(rows.sum())} rows, max|d| elsewhere "
            f"{d:.3e}")
        assert d <= 2e-3
    assert torch.equal(lse[:, rows], glse[:, rows])
    own = torch.ones(N, dtype=torch.bool, device="cuda")
    own[list(prow)] = False
    own &= rows
    for name, a, b in (("dk", dk, gdk), ("dv", dv, gdv)):
        assert torch.equal(a[own], b[own]), name
        d = (a[~own] - b[~own]).abs().max().item()
        say(f"  {name}: bitwise on {int(own.sum())} rows, max|d| on the "
            f"rest {d:.3e}")
        assert d <= 2e-3
