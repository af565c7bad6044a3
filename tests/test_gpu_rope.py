"""GPU parity of the RoPE prologue (rotation at global positions, linear
position interpolation) against the float64 oracle, and of S²-Attn with
RoPE inside the autograd op, end to end."""
import numpy as np
import pytest
import torch

import oracle
import synthetic as syn
from oracle.rope import pair_index
from gpu_helpers import compare, compare_lse, say, scale_for, to_dev

pytestmark = pytest.mark.gpu

s2a = pytest.importorskip("sparse_attention_long_attn_amd")

PAIR = {oracle.HALF: "half", oracle.INTERLEAVED: "interleaved"}


def bf16_round(x64: np.ndarray) -> np.ndarray:
    """float64 -> nearest bf16 (via float32), widened back to float64."""
    return syn.bf16_bits_to_f64(syn.f32_to_bf16_bits(x64.astype(np.float32)))


# B, N, H, D, base, pos_scale, position kind
CASES = [
    (1, 64, 4, 16, 10000.0, 1.0, "none"),
    (2, 300, 3, 32, 10000.0, 0.25, "random"),
    (1, 1024, 4, 64, 500000.0, 1.0, "none"),
    (1, 4096, 2, 128, 10000.0, 1.0, "none"),
    (2, 512, 8, 128, 10000.0, 1.0 / 32, "large"),
]


def positions(kind, B, N, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    if kind == "none":
        return None
    if kind == "random":
        return g.integers(-1000, 100000, (B, N)).astype(np.int32)
    return (g.integers(0, 1 << 20, (B, N))).astype(np.int32)   # up to 1e6


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c)))
@pytest.mark.parametrize("pairing", [oracle.HALF, oracle.INTERLEAVED])
def test_rope_parity(case, pairing):
    B, N, H, D, base, ps, kind = case
    i = CASES.index(case)
    bits = syn.normal_bf16_bits(700 + i, (B, N, H, D))
    pos = positions(kind, B, N, 710 + i)
    say(f"rope B={B} N={N} H={H} D={D} base={base} pos_scale={ps} "
        f"positions={kind} pairing={PAIR[pairing]}")
    x = to_dev(bits)
    pd = None if pos is None else torch.from_numpy(pos).cuda()
    y = s2a.rope(x, base=base, pos_scale=ps, pos_ids=pd,
                 pairing=PAIR[pairing])
    torch.cuda.synchronize()
    want = oracle.rope(syn.bf16_bits_to_f64(bits), base=base, pos_scale=ps,
                       pos_ids=pos, pairing=pairing)
    got = y.float().cpu().numpy().astype(np.float64)
    # y is the fp32 rotation rounded once to bf16.  The fp32 rotation is off
    # by at most e32 = 4 * 2^-24 * (|x_a| + |x_b|) (cos, sin and two products
    # rounded), which matters where the rotated value nearly cancels; the
    # bf16 rounding adds half an ulp, at most 2^-8 relative.
    a_i, b_i = pair_index(D, pairing)
    r = np.sqrt(want[..., a_i] ** 2 + want[..., b_i] ** 2)  # pair norms
    e32 = np.empty_like(want)
    e32[..., a_i] = e32[..., b_i] = 4 * 2.0 ** -24 * np.sqrt(2.0) * r
    err = np.abs(got - want)
    bound = 2.0 ** -8 * (np.abs(want) + e32) + e32
    exact = float(np.mean(got == bf16_round(want)))
    say(f"  max rel err {float(np.max(err / (np.abs(want) + 1e-30))):.3e}, "
        f"equal to bf16(exact) {exact:.5f}")
    assert np.all(err <= bound)
    assert exact >= 0.995
    # in place gives the same bits
    x2 = x.clone()
    s2a.rope(x2, base=base, pos_scale=ps, pos_ids=pd, pairing=PAIR[pairing],
             out=x2)
    torch.cuda.synchronize()
    assert torch.equal(x2, y)
    # the gradient map R^T on float32
    g = torch.from_numpy(syn.normal_f32(720 + i, (B, N, H, D))).cuda()
    gx = s2a.rope_bwd(g, base=base, pos_scale=ps, pos_ids=pd,
                      pairing=PAIR[pairing])
    torch.cuda.synchronize()
    gwant = oracle.rope(g.cpu().numpy().astype(np.float64), base=base,
                        pos_scale=ps, pos_ids=pos, pairing=pairing,
                        inverse=True)
    gerr = float(np.max(np.abs(gx.cpu().numpy() - gwant)))
    say(f"  rope_bwd max abs err {gerr:.3e}")
    assert gerr <= 4e-6


def test_rope_default_positions_equal_explicit_indices():
    B, N, H, D = 2, 256, 4, 64
    x = to_dev(syn.normal_bf16_bits(730, (B, N, H, D)))
    idx = torch.arange(N, dtype=torch.int32, device="cuda").repeat(B, 1)
    a = s2a.rope(x)
    b = s2a.rope(x, pos_ids=idx.contiguous())
    torch.cuda.synchronize()
    assert torch.equal(a, b)


# B, N, H, D, G, L, boundary, positions
ATT_CASES = [
    (1, 1024, 4, 128, 256, 1000, syn.WRAP, "global"),
    (1, 1024, 4, 128, 256, 1024, syn.SPLIT, "global"),
    (1, 768, 4, 64, 384, 700, syn.CYCLIC, "global"),
    (1, 2048, 2, 128, 512, 2000, syn.WRAP, "interp"),
    (2, 640, 4, 32, 320, 600, syn.WRAP, "documents"),
]


@pytest.mark.parametrize("case", ATT_CASES,
                         ids=lambda c: "x".join(map(str, c)))
def test_attention_with_rope_end_to_end(case):
    # Unrotated q, k: the prologue rotates them at their global positions,
    # the attention runs on the rotated tensors, and dq, dk are rotated back
    # by R^T.  The oracle rotates in float64, rounds to bf16 as the prologue
    # does, and runs its float64 attention.
    B, N, H, D, G, L, boundary, kind = case
    i = ATT_CASES.index(case)
    bits = syn.make_inputs(800 + i, boundary, B, N, H, D, with_do=True, L=L)
    base, ps, pos, doc = 10000.0, 1.0, None, None
    if kind == "interp":
        ps = 0.125      # L0 / L1 = 4K / 32K
    if kind == "documents":
        doc = syn.make_doc_ids(810 + i, B, N, 120, cuts=(G // 2, G))
        pos = syn.doc_positions(doc)
    sc = scale_for(D)
    say(f"rope+attention B={B} N={N} H={H} D={D} G={G} L={L} "
        f"boundary={boundary} positions={kind}")
    q, k, v, do = (to_dev(bits[t]) for t in ("q", "k", "v", "do"))
    cfg = dict(base=base, pos_scale=ps, pairing="half",
               pos_ids=None if pos is None else torch.from_numpy(pos).cuda())
    dd = None if doc is None else torch.from_numpy(doc).cuda()
    kw = dict(G=G, boundary=boundary, valid_len=L, scale=sc, doc_ids=dd)
    qr, kr = s2a.rope(q, **cfg), s2a.rope(k, **cfg)
    o, lse = s2a.fwd(qr, kr, v, **kw)
    dq, dk, dv = s2a.bwd(qr, kr, v, o, lse, do, **kw)
    s2a.rope_bwd(dq, out=dq, **cfg)
    s2a.rope_bwd(dk, out=dk, **cfg)
    torch.cuda.synchronize()

    qf, kf, vf, dof = (syn.bf16_bits_to_f64(bits[t]) for t in ("q", "k", "v", "do"))
    rq = bf16_round(oracle.rope(qf, base=base, pos_scale=ps, pos_ids=pos))
    rk = bf16_round(oracle.rope(kf, base=base, pos_scale=ps, pos_ids=pos))
    rdq, rdk, rdv, ro, rlse = oracle.backward(rq, rk, vf, dof, G, G // 2,
                                              boundary, L, sc, doc=doc)
    rdq = oracle.rope(rdq, base=base, pos_scale=ps, pos_ids=pos, inverse=True)
    rdk = oracle.rope(rdk, base=base, pos_scale=ps, pos_ids=pos, inverse=True)
    compare("o", o.cpu().numpy(), ro, valid_rows=L)
    compare_lse(lse.cpu().numpy(), rlse, L)
    compare("dq", dq.cpu().numpy(), rdq, valid_rows=L)
    compare("dk", dk.cpu().numpy(), rdk, valid_rows=L)
    compare("dv", dv.cpu().numpy(), rdv, valid_rows=L)

    # the autograd op does exactly this composition (gradients come back in
    # the inputs' dtype), with either backward
    qa, ka, va = (t.clone().requires_grad_(True) for t in (q, k, v))
    oa = s2a.s2_attention(qa, ka, va, G, boundary=boundary, valid_len=L,
                          scale=sc, doc_ids=dd, rope_cfg=cfg,
                          backward="recompute")
    oa.backward(do.float())
    torch.cuda.synchronize()
    assert torch.equal(oa, o)
    assert torch.equal(qa.grad, dq.to(torch.bfloat16))
    assert torch.equal(ka.grad, dk.to(torch.bfloat16))
    assert torch.equal(va.grad, dv.to(torch.bfloat16))
    # "auto" takes the stored-dS backward when there is no document mask
    # and D is 64 or 128: dk, dv bit for bit as above, dq from the stored dS
    if dd is None and D in (64, 128):
        kw_ds = {n: x for n, x in kw.items() if n != "doc_ids"}
        dq2, _, _ = s2a.bwd_ds(qr, kr, v, o, lse, do, **kw_ds)
        s2a.rope_bwd(dq2, out=dq2, **cfg)
    else:
        dq2 = dq
    qa, ka, va = (t.clone().requires_grad_(True) for t in (q, k, v))
    oa = s2a.s2_attention(qa, ka, va, G, boundary=boundary, valid_len=L,
                          scale=sc, doc_ids=dd, rope_cfg=cfg)
    oa.backward(do.float())
    torch.cuda.synchronize()
    assert torch.equal(qa.grad, dq2.to(torch.bfloat16))
    assert torch.equal(ka.grad, dk.to(torch.bfloat16))
    assert torch.equal(va.grad, dv.to(torch.bfloat16))
    compare("dq (autograd, auto)", dq2.cpu().numpy(), rdq, valid_rows=L)


@pytest.mark.parametrize("boundary", [syn.WRAP, syn.SPLIT, syn.CYCLIC])
def test_attention_invariant_to_a_global_position_offset(boundary):
    # Logits depend on position differences only ([LL] §3.1), so moving
    # every position ID by the same amount changes the outputs only through
    # the bf16 rounding of the rotated q, k.  A path that rotated by in-group
    # offsets would instead change the wrapped group (WRAP, CYCLIC).
    B, N, H, D, G, L = 1, 2048, 4, 128, 512, 2000
    bits = syn.make_inputs(850, boundary, B, N, H, D, L=L)
    q, k, v = (to_dev(bits[t]) for t in ("q", "k", "v"))
    idx = np.tile(np.arange(N, dtype=np.int32), (B, 1))
    outs = []
    for off in (0, 77777):
        pd = torch.from_numpy(idx + off).cuda()
        qr, kr = s2a.rope(q, pos_ids=pd), s2a.rope(k, pos_ids=pd)
        o, lse = s2a.fwd(qr, kr, v, G=G, boundary=boundary, valid_len=L)
        outs.append((o, lse))
    torch.cuda.synchronize()
    do_ = (outs[0][0] - outs[1][0]).abs()
    dl = (outs[0][1][..., :L] - outs[1][1][..., :L]).abs()
    say(f"  offset change: o max {do_.max().item():.3e} mean "
        f"{do_.mean().item():.3e}, lse max {dl.max().item():.3e}")
    # each run is within the parity bound (1e-2) of the same exact result
    assert do_.max().item() <= 2e-2 and do_.mean().item() <= 1e-3
    assert dl.max().item() <= 2e-2
