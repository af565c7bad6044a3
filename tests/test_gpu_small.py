"""GPU parity against the float64 oracle at sizes the oracle finishes in
seconds: every output element is compared.  Cases span several tiles,
ragged valid lengths, both boundary variants, shift 0 and G/2, G = N, and
every supported head width."""
import numpy as np
import pytest
import torch

import oracle
import synthetic as syn
from gpu_helpers import (ATOL_MAX, compare, compare_lse, heads_f64, say,
                         scale_for, to_dev)

pytestmark = pytest.mark.gpu

s2a = pytest.importorskip("sparse_attention_long_attn_amd")

BNAME = {syn.WRAP: "wrap", syn.SPLIT: "split", syn.CYCLIC: "cyclic"}

# B, N, H, D, G, L, half(shift = half*G/2)
CASES = [
    (1, 64, 4, 16, 16, 64, 1),        # the tiny workload
    (1, 8, 2, 16, 4, 8, 1),           # the N=8, G=4 worked example
    (1, 8, 2, 16, 4, 5, 1),
    (1, 8, 2, 16, 4, 1, 1),
    (1, 16, 2, 16, 4, 13, 1),
    (2, 768, 4, 64, 384, 700, 1),     # several tiles, ragged tail
    (1, 1024, 4, 128, 256, 1000, 1),
    (1, 1024, 2, 128, 1024, 1024, 1),  # G = N: full causal
    (1, 640, 4, 32, 320, 555, 1),
    (1, 512, 4, 128, 128, 512, 0),    # shift 0: plain grouping
    (1, 4096, 2, 128, 1024, 3999, 1),
    (1, 2304, 2, 128, 384, 2250, 1),   # groups not a multiple of 256 rows
    (2, 192, 2, 128, 96, 190, 1),      # groups shorter than one key tile
    (1, 8192, 2, 128, 2048, 8000, 1),  # many tiles per group, padded
]


def run_case(B, N, H, D, G, L, half, boundary, seed, with_bwd):
    shift = half * G // 2
    bits = syn.make_inputs(90 + seed, boundary, B, N, H, D, with_do=True, L=L)
    q, k, v, do = (to_dev(bits[t]) for t in ("q", "k", "v", "do"))
    sc = scale_for(D)
    say(f"case B={B} N={N} H={H} D={D} G={G} L={L} shift={shift} "
        f"{BNAME[boundary]} bwd={with_bwd}")
    o, lse = s2a.fwd(q, k, v, G=G, shift=shift, boundary=boundary,
                     valid_len=L, scale=sc)
    torch.cuda.synchronize()
    qf, kf, vf, dof = (syn.bf16_bits_to_f64(bits[t]) for t in ("q", "k", "v", "do"))
    if with_bwd:
        dq, dk, dv = s2a.bwd(q, k, v, o, lse, do, G=G, shift=shift,
                             boundary=boundary, valid_len=L, scale=sc)
        torch.cuda.synchronize()
        rdq, rdk, rdv, ro, rlse = oracle.backward(qf, kf, vf, dof, G, shift,
                                                  boundary, L, sc)
    else:
        ro, rlse = oracle.forward(qf, kf, vf, G, shift, boundary, L, sc)
    compare("o", o.cpu().numpy(), ro, valid_rows=L)
    compare_lse(lse.cpu().numpy(), rlse, L)
    if with_bwd:
        compare("dq", dq.cpu().numpy(), rdq, valid_rows=L)
        compare("dk", dk.cpu().numpy(), rdk, valid_rows=L)
        compare("dv", dv.cpu().numpy(), rdv, valid_rows=L)


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c)))
@pytest.mark.parametrize("boundary", [syn.WRAP, syn.SPLIT, syn.CYCLIC])
def test_forward_backward_small(case, boundary):
    run_case(*case, boundary=boundary, seed=CASES.index(case),
             with_bwd=True)


MAP_CASES = [(8, 4), (16, 4), (64, 16), (48, 12), (12, 12), (24, 2),
             (8192, 2048), (32768, 8192), (12288, 12288), (12288, 6144),
             (12288, 3072), (12288, 2048), (12288, 1536), (102400, 25600)]


@pytest.mark.parametrize("N,G", MAP_CASES)
@pytest.mark.parametrize("boundary", [syn.WRAP, syn.SPLIT, syn.CYCLIC])
@pytest.mark.parametrize("half", [0, 1])
def test_group_map_bit_exact(N, G, boundary, half):
    shift = half * G // 2
    gid, slot, src = s2a.group_map(N, G, shift=shift, boundary=boundary,
                                   valid_len=N)
    torch.cuda.synchronize()
    ref = oracle.group_maps_a(N, G, shift, boundary)
    for name, got, want in zip(("gid", "slot", "src"), (gid, slot, src), ref):
        assert np.array_equal(got.cpu().numpy(), want), name


def test_forward_bitwise_repeatable():
    B, N, H, D, G = 1, 2048, 4, 128, 512
    bits = syn.make_inputs(77, 0, B, N, H, D)
    q, k, v = (to_dev(bits[t]) for t in ("q", "k", "v"))
    o1, l1 = s2a.fwd(q, k, v, G=G, boundary="wrap")
    o2, l2 = s2a.fwd(q, k, v, G=G, boundary="wrap")
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_bf16_output_option():
    B, N, H, D, G, L = 1, 1024, 4, 128, 256, 1000
    bits = syn.make_inputs(78, 0, B, N, H, D)
    q, k, v = (to_dev(bits[t]) for t in ("q", "k", "v"))
    o, lse = s2a.fwd(q, k, v, G=G, boundary="split", valid_len=L,
                     out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    qf, kf, vf = (syn.bf16_bits_to_f64(bits[t]) for t in ("q", "k", "v"))
    ro, rlse = oracle.forward(qf, kf, vf, G, G // 2, syn.SPLIT, L, scale_for(D))
    # bf16 output adds at most half a bf16 ulp (2^-6 for |o| < 8)
    compare("o_bf16", o.float().cpu().numpy(), ro, valid_rows=L,
            atol_max=ATOL_MAX + 2.0 ** -6)
    compare_lse(lse.cpu().numpy(), rlse, L)


@pytest.mark.parametrize("boundary", [syn.WRAP, syn.SPLIT])
def test_forward_large_logit_growth(boundary):
    # Keys from slot 100 of every group on are scaled by 30, so a row's
    # running max grows by far more than the forward's lazy-rescale
    # threshold after its first key blocks: the O rescale path must run.
    B, N, H, D, G, L = 1, 1024, 2, 128, 512, 1000
    bits = syn.make_inputs(77, boundary, B, N, H, D)
    kf = syn.bf16_bits_to_f64(bits["k"]).astype(np.float32)
    slot = np.arange(N) % G
    kf[:, slot >= 100] *= 30.0
    kbits = syn.f32_to_bf16_bits(kf)
    q, k, v = to_dev(bits["q"]), to_dev(kbits), to_dev(bits["v"])
    sc = scale_for(D)
    o, lse = s2a.fwd(q, k, v, G=G, boundary=boundary, valid_len=L, scale=sc)
    torch.cuda.synchronize()
    qf, vf = syn.bf16_bits_to_f64(bits["q"]), syn.bf16_bits_to_f64(bits["v"])
    ro, rlse = oracle.forward(qf, syn.bf16_bits_to_f64(kbits), vf, G, G // 2,
                              boundary, L, sc)
    assert np.nanmax(rlse[..., :L]) > 40.0   # the growth really happened
    # With a near one-hot softmax the bf16 rounding of P (2^-9 relative)
    # no longer averages out: |dO| <= 2^-9 max|v| + 2^-9 |O| (numerator and
    # normaliser), so the bound is 2^-8 max|v|.  A missing or wrong rescale
    # would be off by factors of 2^60, not by 1e-2.
    tol = 2.0 ** -8 * float(np.abs(vf).max())
    compare("o", o.cpu().numpy(), ro, valid_rows=L, atol_max=tol)
    compare_lse(lse.cpu().numpy(), rlse, L)


def test_invalid_arguments_write_nothing():
    B, N, H, D, G = 1, 64, 4, 16, 16
    q = torch.zeros((B, N, H, D), dtype=torch.bfloat16, device="cuda")
    o = torch.full((B, N, H, D), 7.0, device="cuda")
    lse = torch.full((B, H, N), 7.0, device="cuda")
    for kw in (dict(G=15), dict(G=16, shift=4), dict(G=16, valid_len=0),
               dict(G=16, valid_len=65), dict(G=24), dict(G=16, scale=-1.0)):
        with pytest.raises(ValueError):
            s2a.fwd(q, q, q, o=o, lse=lse, **kw)
    torch.cuda.synchronize()
    assert torch.all(o == 7.0) and torch.all(lse == 7.0)
