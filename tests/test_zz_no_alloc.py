"""The no-allocation backward (s2attn_bwd_noalloc): the same results as
s2attn_bwd bit for bit, with its delta array kept by the library on the
device.  Two calls in a row, the second smaller, so the second reuses the
array the first filled; one case is also checked against the oracle."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import synthetic as syn
from gpu_helpers import compare, say, scale_for, to_dev

pytestmark = pytest.mark.gpu

s2a = pytest.importorskip("sparse_attention_long_attn_amd")
from sparse_attention_long_attn_amd import _lib  # noqa: E402


def _noalloc_call(q, k, v, o, lse, do, dq, dk, dv, G, boundary, L, sc):
    """Straight through the C ABI (ctypes), with preallocated outputs."""
    B, N, H, D = q.shape
    st = _lib.load().s2attn_bwd_noalloc(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), _lib.S2A_F32,
        lse.data_ptr(), do.data_ptr(), dq.data_ptr(), dk.data_ptr(),
        dv.data_ptr(), B, N, H, D, G, G // 2, boundary, L, None, sc,
        torch.cuda.current_stream().cuda_stream)
    assert st == 0, _lib.load().s2attn_last_error().decode()


@pytest.mark.parametrize("boundary", [syn.WRAP, syn.SPLIT])
def test_noalloc_backward_equals_backward(boundary):
    # the second call is smaller: it must not see the first call's delta
    cases = [(2, 4096, 8, 128, 1024, 4000), (1, 768, 4, 64, 256, 700)]
    for i, (B, N, H, D, G, L) in enumerate(cases):
        say(f"no-alloc call {i}: B={B} N={N} H={H} D={D} G={G} L={L} "
            f"boundary={boundary}")
        bits = syn.make_inputs(300 + i, boundary, B, N, H, D, with_do=True,
                               L=L)
        q, k, v, do = (to_dev(bits[t]) for t in ("q", "k", "v", "do"))
        sc = scale_for(D)
        kw = dict(G=G, boundary=boundary, valid_len=L, scale=sc)
        o, lse = s2a.fwd(q, k, v, **kw)
        dq0, dk0, dv0 = s2a.bwd(q, k, v, o, lse, do, **kw)
        dq, dk, dv = (torch.full_like(dq0, float("nan")) for _ in range(3))
        _noalloc_call(q, k, v, o, lse, do, dq, dk, dv, G, boundary, L, sc)
        torch.cuda.synchronize()
        assert torch.equal(dq, dq0) and torch.equal(dk, dk0) \
            and torch.equal(dv, dv0)
        if i == 1:
            f = [syn.bf16_bits_to_f64(bits[t]) for t in ("q", "k", "v", "do")]
            rdq, rdk, rdv, _, _ = oracle.backward(*f, G, G // 2, boundary, L,
                                                  sc)
            compare("dq (no-alloc)", dq.cpu().numpy(), rdq, valid_rows=L)
            compare("dk (no-alloc)", dk.cpu().numpy(), rdk, valid_rows=L)
            compare("dv (no-alloc)", dv.cpu().numpy(), rdv, valid_rows=L)


def test_noalloc_rejects_more_rows_than_it_holds():
    B, N, H, D, G = 1, 1 << 20, 8, 64, 1024   # B*H*N = 2^23 > 2^22
    q = torch.zeros((1, 16, 2, 16), dtype=torch.bfloat16, device="cuda")
    out = torch.full((16,), 7.0, device="cuda")
    p = q.data_ptr()
    st = _lib.load().s2attn_bwd_noalloc(p, p, p, p, _lib.S2A_BF16, p, p,
                                        out.data_ptr(), p, p, B, N, H, D, G,
                                        G // 2, syn.WRAP, N, None, 0.125, None)
    assert st == _lib.S2A_EINVAL
    assert "no-allocation" in _lib.load().s2attn_last_error().decode()
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)
