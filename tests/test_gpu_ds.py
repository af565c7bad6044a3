"""GPU parity of the backward that stores dS (s2attn_bwd_ds) against the
float64 oracle at sizes the oracle finishes in seconds, every element
compared.  Its dK/dV stage is the recompute path's kernel plus the dS
stores, so dk and dv must equal s2attn_bwd's bit for bit; dq is summed
from the stored bf16 dS and must meet the same tolerance as s2attn_bwd.
The workspace starts as garbage (0xFF bytes, NaN in bf16): no output may
depend on workspace bytes the dK/dV stage did not write."""
import numpy as np
import pytest
import torch

import oracle
import synthetic as syn
from gpu_helpers import compare, say, scale_for, to_dev

pytestmark = pytest.mark.gpu

s2a = pytest.importorskip("sparse_attention_long_attn_amd")

BNAME = {syn.WRAP: "wrap", syn.SPLIT: "split", syn.CYCLIC: "cyclic"}

# B, N, H, D, G, L, half (shift = half * G / 2)
CASES = [
    (2, 768, 4, 64, 384, 700, 1),      # several tiles, ragged tail
    (1, 1024, 4, 128, 256, 1000, 1),
    (1, 1024, 2, 128, 1024, 1024, 1),  # G = N: full causal
    (1, 512, 4, 128, 128, 512, 0),     # shift 0
    (1, 4096, 2, 128, 1024, 3999, 1),
    (1, 2304, 2, 128, 384, 2250, 1),   # groups not a multiple of 256 rows
    (2, 192, 2, 128, 96, 190, 1),      # groups shorter than one key block
    (1, 256, 2, 64, 64, 256, 1),       # half groups of 32 slots
    (1, 8, 2, 64, 4, 5, 1),            # the N=8, G=4 worked example, padded
    (1, 8192, 2, 128, 2048, 8000, 1),  # many key blocks per group, padded
    (1, 16, 2, 64, 2, 13, 1),          # groups of two tokens (s = 1)
    (2, 64, 4, 64, 32, 50, 0),         # shift 0, padded, B = 2
    (1, 384, 2, 128, 384, 200, 1),     # G = N (no shift), half padded
]


def _inputs(case, boundary, seed):
    B, N, H, D, G, L, half = case
    bits = syn.make_inputs(95 + seed, boundary, B, N, H, D, with_do=True, L=L)
    return bits, [to_dev(bits[t]) for t in ("q", "k", "v", "do")]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c)))
@pytest.mark.parametrize("boundary", [syn.WRAP, syn.SPLIT, syn.CYCLIC])
def test_stored_ds_backward(case, boundary):
    B, N, H, D, G, L, half = case
    shift = half * G // 2
    sc = scale_for(D)
    bits, (q, k, v, do) = _inputs(case, boundary, CASES.index(case))
    say(f"stored-dS case B={B} N={N} H={H} D={D} G={G} L={L} shift={shift} "
        f"{BNAME[boundary]}")
    kw = dict(G=G, shift=shift, boundary=boundary, valid_len=L, scale=sc)
    o, lse = s2a.fwd(q, k, v, **kw)
    dq0, dk0, dv0 = s2a.bwd(q, k, v, o, lse, do, **kw)
    ws = s2a.ds_workspace(q, G=G, shift=shift, boundary=boundary)
    ws.fill_(255)
    dq, dk, dv = s2a.bwd_ds(q, k, v, o, lse, do, ds_ws=ws, **kw)
    torch.cuda.synchronize()
    assert torch.equal(dk, dk0) and torch.equal(dv, dv0)
    qf, kf, vf, dof = (syn.bf16_bits_to_f64(bits[t]) for t in ("q", "k", "v", "do"))
    rdq, rdk, rdv, _, _ = oracle.backward(qf, kf, vf, dof, G, shift,
                                          boundary, L, sc)
    compare("dq (stored dS)", dq.cpu().numpy(), rdq, valid_rows=L)
    compare("dk", dk.cpu().numpy(), rdk, valid_rows=L)
    compare("dv", dv.cpu().numpy(), rdv, valid_rows=L)
    dd = (dq - dq0).abs().max().item()
    say(f"  dq vs recompute path: max|d|={dd:.3e}")
    # a second call over the same (now written) workspace, zeroed first:
    # bit for bit the same
    ws.zero_()
    dq2, dk2, dv2 = s2a.bwd_ds(q, k, v, o, lse, do, ds_ws=ws, **kw)
    torch.cuda.synchronize()
    assert torch.equal(dq2, dq) and torch.equal(dk2, dk) and torch.equal(dv2, dv)


def test_stored_ds_stages_equal_whole_call():
    B, N, H, D, G, L = 1, 2048, 4, 128, 512, 2000
    bits, (q, k, v, do) = _inputs((B, N, H, D, G, L, 1), syn.WRAP, 40)
    kw = dict(G=G, boundary=syn.WRAP, valid_len=L)
    o, lse = s2a.fwd(q, k, v, **kw)
    ws = s2a.ds_workspace(q, G=G)
    dq, dk, dv = s2a.bwd_ds(q, k, v, o, lse, do, ds_ws=ws, **kw)
    delta = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    dq1, dk1, dv1 = (torch.full_like(dq, float("nan")) for _ in range(3))
    ws.fill_(255)
    s2a.bwd_preprocess(o, do, delta)
    s2a.bwd_dkdv_ds(q, k, v, lse, delta, do, dk1, dv1, ws, **kw)
    s2a.bwd_dq_ds(k, ws, dq1, **kw)
    torch.cuda.synchronize()
    assert torch.equal(dq1, dq) and torch.equal(dk1, dk) and torch.equal(dv1, dv)


def test_stored_ds_rejects_what_it_does_not_cover():
    q = torch.zeros((1, 64, 2, 32), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(Exception, match="D in"):
        s2a.ds_workspace(q, G=16)
    q = torch.zeros((1, 256, 2, 128), dtype=torch.bfloat16, device="cuda")
    o = torch.zeros((1, 256, 2, 128), dtype=torch.float32, device="cuda")
    lse = torch.zeros((1, 2, 256), dtype=torch.float32, device="cuda")
    need = s2a.ds_workspace_bytes(1, 256, 2, 128, G=64)
    short = torch.zeros(need - 16, dtype=torch.uint8, device="cuda")
    dq = torch.full_like(o, 7.0)
    with pytest.raises(Exception, match="workspace"):
        s2a.bwd_ds(q, q, q, o, lse, q, G=64, ds_ws=short, dq=dq)
    torch.cuda.synchronize()
    assert torch.all(dq == 7.0)  # nothing written


def test_host_buffers_rejected_before_launch():
    # Every tensor argument of the torch wrappers must sit on q's GPU: a
    # host tensor (whose pointer a kernel would dereference) is a
    # ValueError before anything is enqueued.
    B, N, H, D, G = 1, 256, 2, 128, 64
    dev = torch.device("cuda")
    q = torch.zeros((B, N, H, D), dtype=torch.bfloat16, device=dev)
    o = torch.zeros((B, N, H, D), dtype=torch.float32, device=dev)
    lse = torch.zeros((B, H, N), dtype=torch.float32, device=dev)
    delta = torch.zeros((B, H, N), dtype=torch.float32, device=dev)
    ws = s2a.ds_workspace(q, G=G)
    cpu_ws = torch.empty(ws.numel(), dtype=torch.uint8)
    cpu32 = torch.zeros((B, N, H, D), dtype=torch.float32)
    cpu_stat = torch.zeros((B, H, N), dtype=torch.float32)
    sentinel = [torch.full_like(o, 7.0) for _ in range(3)]
    dq, dk, dv = sentinel
    calls = [
        lambda: s2a.bwd_ds(q, q, q, o, lse, q, G=G, ds_ws=cpu_ws, dq=dq,
                           dk=dk, dv=dv),
        lambda: s2a.bwd_dkdv_ds(q, q, q, lse, delta, q, dk, dv, cpu_ws, G=G),
        lambda: s2a.bwd_dq_ds(q, cpu_ws, dq, G=G),
        lambda: s2a.bwd_dq_ds(q, ws, cpu32, G=G),
        lambda: s2a.bwd_dkdv_ds(q, q, q, lse, delta, q, cpu32, dv, ws, G=G),
        lambda: s2a.bwd_dkdv_ds(q, q, q, cpu_stat, delta, q, dk, dv, ws,
                                G=G),
        lambda: s2a.bwd_dkdv(q, q, q, lse, cpu_stat, q, dk, dv, G=G),
        lambda: s2a.bwd_dq(q, q, q, lse, delta, q, cpu32, G=G),
        lambda: s2a.bwd(q, q, q, o, lse, q, G=G, dq=cpu32, dk=dk, dv=dv),
        lambda: s2a.bwd(q, q, q, o, lse, q, G=G, dq=dq, dk=dk, dv=dv,
                        delta=cpu_stat),
        lambda: s2a.bwd(q, q, q, cpu32, lse, q, G=G, dq=dq, dk=dk, dv=dv),
        lambda: s2a.bwd_preprocess(o, q, cpu_stat),
        lambda: s2a.fwd(q, q, q, G=G, o=cpu32),
        lambda: s2a.fwd(q, q, q, G=G, o=o, lse=cpu_stat),
    ]
    for i, call in enumerate(calls):
        say(f"  host-buffer call {i}")
        with pytest.raises(ValueError):
            call()
    torch.cuda.synchronize()
    for t in sentinel:
        assert torch.all(t == 7.0)  # nothing was written
