"""CPU checks of the C ABI: the library loads without a GPU, exports every
function include/s2attn.h declares, and rejects bad arguments with the
documented status before touching the device.  Also pins the host-side
work accounting against the oracle's enumerated pair counts."""
import ctypes
import os
import re

import pytest

import oracle
from sparse_attention_long_attn_amd import _lib, work

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    text = open(os.path.join(ROOT, "include", "s2attn.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(s2attn_\w+)\s*\(", text)))


def test_header_declares_the_three_entry_points():
    fns = header_functions()
    for name in ("s2attn_fwd", "s2attn_bwd", "s2attn_group_map"):
        assert name in fns


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    for name in header_functions():
        assert hasattr(lib, name), name
    assert set(header_functions()) <= set(_lib.EXPORTS)


NULL = None
OK_ARGS = dict(B=1, N=64, H=4, D=16, G=16, shift=8, boundary=0, L=64,
               scale=0.25)


def call_fwd(**kw):
    a = dict(OK_ARGS, **kw)
    lib = _lib.load()
    return lib.s2attn_fwd(NULL, NULL, NULL, NULL, 1, NULL, a["B"], a["N"],
                          a["H"], a["D"], a["G"], a["shift"], a["boundary"],
                          a["L"], a.get("doc"), a["scale"], NULL)


def call_bwd(**kw):
    a = dict(OK_ARGS, **kw)
    lib = _lib.load()
    return lib.s2attn_bwd(NULL, NULL, NULL, NULL, 1, NULL, NULL, NULL, NULL,
                          NULL, NULL, a["B"], a["N"], a["H"], a["D"], a["G"],
                          a["shift"], a["boundary"], a["L"], a.get("doc"),
                          a["scale"], NULL)


@pytest.mark.parametrize("kw,status", [
    (dict(H=3), _lib.S2A_EINVAL),
    (dict(G=15, shift=7), _lib.S2A_EINVAL),
    (dict(N=60), _lib.S2A_EINVAL),
    (dict(L=0), _lib.S2A_EINVAL),
    (dict(L=65), _lib.S2A_EINVAL),
    (dict(shift=4), _lib.S2A_EINVAL),
    (dict(boundary=3), _lib.S2A_EINVAL),
    (dict(B=0), _lib.S2A_EINVAL),
    (dict(D=24), _lib.S2A_EUNSUPPORTED),
    (dict(D=256), _lib.S2A_EUNSUPPORTED),
    (dict(H=1 << 17, D=128), _lib.S2A_EUNSUPPORTED),   # H*D = 2^24
    (dict(doc=6), _lib.S2A_EINVAL),                    # misaligned doc IDs
    (dict(), _lib.S2A_EINVAL),          # valid shape, NULL pointers
])
@pytest.mark.parametrize("call", [call_fwd, call_bwd])
def test_bad_arguments_rejected_before_launch(kw, status, call):
    assert call(**kw) == status
    assert _lib.load().s2attn_last_error().decode() != ""


def test_misaligned_pointer_rejected():
    lib = _lib.load()
    buf = (ctypes.c_char * 4096)()
    base = ctypes.addressof(buf)
    p = ((base + 15) // 16) * 16
    st = lib.s2attn_fwd(p + 2, p, p, p, 1, p, 1, 64, 4, 16, 16, 8, 0, 64,
                        None, 0.25, None)
    assert st == _lib.S2A_EINVAL
    assert "aligned" in lib.s2attn_last_error().decode()
    st = lib.s2attn_fwd(p, p, p, p, 1, p, 1, 64, 4, 16, 16, 8, 0, 64,
                        None, float("nan"), None)
    assert st == _lib.S2A_EINVAL


def test_stored_ds_workspace_size():
    # blocks of 64 queries x 128 keys (16 KiB): per (b, h, group),
    # nkb (nkb + 1) + 2 with nkb = ceil(len / 128) for the group's length
    # (the causal blocks plus two residual blocks of key block 0).  The
    # group lengths come from the oracle's segments: under SPLIT the shifted
    # class has two groups of length G/2 and one group more.
    import oracle
    lib = _lib.load()
    out = ctypes.c_size_t(0)

    def blocks(n):
        nkb = -(-n // 128)
        return nkb * (nkb + 1) + 2

    for (B, N, H, D, G, bnd) in [(1, 32768, 32, 128, 8192, 0),
                                 (2, 12288, 32, 64, 1536, 1),
                                 (1, 102400, 32, 128, 25600, 1),
                                 (1, 102400, 32, 128, 25600, 2),
                                 (1, 1024, 2, 128, 1024, 2),
                                 (1, 192, 2, 128, 96, 0),
                                 (1, 192, 2, 128, 96, 1),
                                 (2, 1536, 6, 64, 512, 1)]:
        for shift in (G // 2, 0):
            assert lib.s2attn_bwd_ds_workspace(B, N, H, D, G, shift, bnd,
                                               ctypes.byref(out)) == _lib.S2A_OK
            segs = oracle.segments(N, G, shift, bnd)
            want = B * sum(blocks(len(seg)) for h in range(H)
                           for seg in segs[int(h >= H // 2)])
            assert out.value == want * 16384, (B, N, H, G, bnd, shift)
    # SPLIT no longer sizes every unit as a full group: at 100K (G = 25600)
    # it needs a quarter less than before
    lib.s2attn_bwd_ds_workspace(1, 102400, 32, 128, 25600, 12800, 1,
                                ctypes.byref(out))
    full = 32 * 5 * blocks(25600) * 16384
    assert out.value < 0.76 * full
    assert lib.s2attn_bwd_ds_workspace(1, 64, 4, 32, 16, 8, 0,
                                       ctypes.byref(out)) == _lib.S2A_EUNSUPPORTED
    assert lib.s2attn_bwd_ds_workspace(1, 64, 4, 64, 16, 8, 0,
                                       None) == _lib.S2A_EINVAL
    assert lib.s2attn_bwd_ds_workspace(1, 60, 4, 64, 16, 8, 0,
                                       ctypes.byref(out)) == _lib.S2A_EINVAL


def test_stored_ds_rejects_bad_workspace_before_launch():
    lib = _lib.load()
    buf = (ctypes.c_char * 4096)()
    p = ((ctypes.addressof(buf) + 15) // 16) * 16
    out = ctypes.c_size_t(0)
    lib.s2attn_bwd_ds_workspace(1, 256, 2, 128, 64, 32, 0, ctypes.byref(out))
    need = out.value

    def ds(ws, nbytes, D=128):
        return lib.s2attn_bwd_ds(p, p, p, p, 1, p, p, p, p, p, p, ws, nbytes,
                                 1, 256, 2, D, 64, 32, 0, 256, 0.1, None)

    def dkdv(ws, nbytes, D=128):
        return lib.s2attn_bwd_dkdv_ds(p, p, p, p, p, p, p, p, ws, nbytes, 1,
                                      256, 2, D, 64, 32, 0, 256, 0.1, None)

    def dq(ws, nbytes, D=128):
        return lib.s2attn_bwd_dq_ds(p, ws, nbytes, p, 1, 256, 2, D, 64, 32, 0,
                                    256, 0.1, None)

    for call in (ds, dkdv, dq):
        assert call(None, need) == _lib.S2A_EINVAL
        assert call(p + 8, need) == _lib.S2A_EINVAL          # misaligned
        assert call(p, need - 1) == _lib.S2A_EINVAL          # too short
        assert "workspace" in lib.s2attn_last_error().decode()
        assert call(p, need, D=32) == _lib.S2A_EUNSUPPORTED


def test_rope_rejects_bad_arguments():
    lib = _lib.load()
    buf = (ctypes.c_char * 4096)()
    p = ((ctypes.addressof(buf) + 15) // 16) * 16
    ok = dict(x=p, y=p, B=1, N=4, H=2, D=16, pos=None, base=10000.0,
              ps=1.0, pairing=0)
    bad = [
        dict(x=None), dict(y=p + 8), dict(B=0), dict(D=24),
        dict(D=256), dict(pos=p + 2), dict(base=0.0),
        dict(base=float("inf")), dict(ps=-1.0), dict(ps=float("nan")),
        dict(pairing=2),
    ]
    for fn in (lib.s2attn_rope, lib.s2attn_rope_bwd):
        for kw in bad:
            a = dict(ok, **kw)
            st = fn(a["x"], a["y"], a["B"], a["N"], a["H"], a["D"], a["pos"],
                    a["base"], a["ps"], a["pairing"], None)
            want = (_lib.S2A_EUNSUPPORTED if kw.get("D") in (24, 256)
                    else _lib.S2A_EINVAL)
            assert st == want, kw
            assert lib.s2attn_last_error().decode() != ""


def test_group_map_rejects_bad_shapes():
    lib = _lib.load()
    assert lib.s2attn_group_map(60, 16, 8, 0, 60, None, None, None, None) \
        == _lib.S2A_EINVAL
    assert lib.s2attn_group_map(64, 16, 8, 0, 64, None, None, None, None) \
        == _lib.S2A_EINVAL


def test_strerror():
    lib = _lib.load()
    for st in range(4):
        assert lib.s2attn_strerror(st)
    with pytest.raises(ValueError):
        _lib.check(_lib.S2A_EINVAL)
    with pytest.raises(_lib.S2AttnError):
        _lib.check(_lib.S2A_EHIP)


@pytest.mark.parametrize("N,G,L", [(64, 16, 64), (64, 16, 50), (64, 16, 5),
                                   (48, 12, 37), (96, 32, 81), (128, 128, 100),
                                   (256, 64, 200), (256, 64, 250)])
@pytest.mark.parametrize("boundary", [0, 1, 2])
@pytest.mark.parametrize("half", [0, 1])
def test_work_pairs_match_oracle_enumeration(N, G, L, boundary, half):
    shift = half * G // 2
    assert work.allowed_pairs(N, G, shift, boundary, L) == \
        oracle.allowed_pairs(N, G, shift, boundary, L)


@pytest.mark.parametrize("N,G,L,mean", [(64, 16, 64, 5), (64, 16, 50, 20),
                                        (96, 32, 81, 7), (256, 64, 250, 40),
                                        (128, 128, 100, 300)])
@pytest.mark.parametrize("boundary", [0, 1, 2])
@pytest.mark.parametrize("half", [0, 1])
def test_work_doc_pairs_match_oracle_enumeration(N, G, L, mean, boundary,
                                                 half):
    import numpy as np
    import synthetic as syn
    from oracle.s2attn_oracle import _with_docs
    shift = half * G // 2
    doc = syn.make_doc_ids(N + G + mean, 1, N, mean, cuts=(G // 3, G))
    rows = np.arange(N)
    want = tuple(int(_with_docs(oracle.adjacency_block(c, rows, N, G, shift,
                                                       boundary, L),
                                doc, 0, rows, np.arange(N)).sum())
                 for c in (0, 1))
    assert work.doc_pairs(N, G, shift, boundary, L, doc[0]) == want
    one = np.zeros(N, np.int32)
    assert work.doc_pairs(N, G, shift, boundary, L, one) == \
        work.allowed_pairs(N, G, shift, boundary, L)


def test_work_pairs_of_the_headline_workload():
    # N=32768, G=8192, WRAP: both classes M*G*(G+1)/2
    c0, c1 = work.allowed_pairs(32768, 8192, 4096, 0, 32768)
    assert c0 == c1 == 4 * 8192 * 8193 // 2
    fwd, bwd = work.useful_flops(1, 32768, 32, 128, 8192, 4096, 0, 32768)
    assert fwd == 4 * 128 * 16 * (c0 + c1) and bwd == 2.5 * fwd


def test_torch_wrappers_reject_host_tensors():
    # The torch layer refuses tensors in host memory with a ValueError
    # before it reaches the library (no GPU is needed to see it).
    import torch
    from sparse_attention_long_attn_amd import ops
    q = torch.zeros((1, 64, 2, 64), dtype=torch.bfloat16)
    o = torch.zeros((1, 64, 2, 64), dtype=torch.float32)
    lse = torch.zeros((1, 2, 64), dtype=torch.float32)
    ws = torch.zeros(1 << 16, dtype=torch.uint8)
    for call in (lambda: ops.fwd(q, q, q, G=16),
                 lambda: ops.bwd(q, q, q, o, lse, q, G=16),
                 lambda: ops.bwd_dq_ds(q, ws, o, G=16),
                 lambda: ops.bwd_dkdv_ds(q, q, q, lse, lse, q, o, o, ws,
                                         G=16)):
        with pytest.raises(ValueError):
            call()
    # the shared check names the argument, its shape and the device wanted
    with pytest.raises(ValueError, match=r"dq must be a contiguous float32 "
                                         r"\(1, 64, 2, 64\) tensor on cuda"):
        ops._need(o, (1, 64, 2, 64), torch.float32, torch.device("cuda"),
                  "dq")
    with pytest.raises(ValueError, match="ds_ws"):
        ops._ds_arg(ws, torch.device("cuda"))


def test_noalloc_backward_rejects_too_many_rows_before_launch():
    # B*H*N beyond the library's delta array: S2A_EINVAL from the host
    # checks alone (the pointers below are never dereferenced)
    lib = _lib.load()
    fake = 1 << 12                      # aligned, never touched
    B, N, H, D, G = 1, 1 << 20, 8, 64, 1024
    assert B * H * N > _lib.S2A_NOALLOC_MAX_ROWS
    st = lib.s2attn_bwd_noalloc(fake, fake, fake, fake, _lib.S2A_F32, fake,
                                fake, fake, fake, fake, B, N, H, D, G,
                                G // 2, _lib.S2A_WRAP, N, None, 0.125, None)
    assert st == _lib.S2A_EINVAL
    assert "no-allocation" in lib.s2attn_last_error().decode()
    # the limit the header states is the one the library enforces
    hdr = open(os.path.join(ROOT, "include", "s2attn.h")).read()
    m = re.search(r"#define S2A_NOALLOC_MAX_ROWS \(1 << (\d+)\)", hdr)
    assert m and (1 << int(m.group(1))) == _lib.S2A_NOALLOC_MAX_ROWS
