"""Thin torch-facing wrappers of the C ABI: argument marshalling only.

Every step of the computation runs in the HIP library; torch provides the
device memory and the current stream.  Nothing here computes attention,
and there is no CPU fallback: without the built library these functions
raise.
"""
from __future__ import annotations

import ctypes
import math

import torch

from . import _lib

BOUNDARIES = {"wrap": _lib.S2A_WRAP, "split": _lib.S2A_SPLIT,
              "cyclic": _lib.S2A_CYCLIC, _lib.S2A_WRAP: _lib.S2A_WRAP,
              _lib.S2A_SPLIT: _lib.S2A_SPLIT, _lib.S2A_CYCLIC: _lib.S2A_CYCLIC}


def _boundary(b) -> int:
    try:
        return BOUNDARIES[b]
    except KeyError:
        raise ValueError(f"boundary must be 'wrap', 'split' or 'cyclic', "
                         f"got {b!r}")


def _ptr(t: torch.Tensor) -> int:
    return t.data_ptr()


def _check_qkv(*ts, shape=None):
    shape = shape or ts[0].shape
    if len(shape) != 4:
        raise ValueError("q, k, v must be [B, N, H, D]")
    for t in ts:
        if t.dtype != torch.bfloat16:
            raise ValueError("q, k, v, dout must be bfloat16")
        if t.shape != shape:
            raise ValueError(f"shape mismatch: {tuple(t.shape)} vs {tuple(shape)}")
        if not t.is_cuda:
            raise ValueError("tensors must be on the GPU")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
    return shape


def _need(t, shape, dtypes, dev, name):
    """Raise ValueError unless ``t`` is a contiguous tensor of ``shape``,
    one of ``dtypes``, on device ``dev`` (checked before any launch: a
    pointer to host memory handed to a kernel faults the GPU)."""
    if not isinstance(dtypes, tuple):
        dtypes = (dtypes,)
    if not isinstance(t, torch.Tensor) or t.dtype not in dtypes \
            or tuple(t.shape) != tuple(shape) or not t.is_contiguous() \
            or t.device != dev:
        names = "/".join(str(d).replace("torch.", "") for d in dtypes)
        raise ValueError(f"{name} must be a contiguous {names} "
                         f"{tuple(shape)} tensor on {dev}")
    return t


def _stream(dev) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def _docs(doc_ids, q):
    """Device pointer of optional int32 [B, N] document IDs (None: none)."""
    if doc_ids is None:
        return None
    B, N = q.shape[0], q.shape[1]
    if doc_ids.dtype != torch.int32 or tuple(doc_ids.shape) != (B, N) \
            or not doc_ids.is_contiguous() or doc_ids.device != q.device:
        raise ValueError("doc_ids must be a contiguous int32 [B, N] tensor on "
                         "the device of q")
    return doc_ids.data_ptr()


def fwd(q, k, v, *, G: int, shift: int | None = None, boundary="wrap",
        valid_len: int | None = None, scale: float | None = None,
        out_dtype=torch.float32, o=None, lse=None, doc_ids=None):
    """S²-Attn forward.  Returns (o [B,N,H,D], lse [B,H,N] float32).
    doc_ids: optional int32 [B, N] document IDs of packed samples."""
    B, N, H, D = _check_qkv(q, k, v)
    shift = G // 2 if shift is None else shift
    valid_len = N if valid_len is None else valid_len
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("out_dtype must be float32 or bfloat16")
    if o is None:
        o = torch.empty((B, N, H, D), dtype=out_dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _need(o, q.shape, out_dtype, q.device, "o")
    _need(lse, (B, H, N), torch.float32, q.device, "lse")
    odt = _lib.S2A_F32 if out_dtype == torch.float32 else _lib.S2A_BF16
    lib = _lib.load()
    _lib.check(lib.s2attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), odt,
                              _ptr(lse), B, N, H, D, G, shift,
                              _boundary(boundary), valid_len,
                              _docs(doc_ids, q), scale, _stream(q.device)))
    return o, lse


def _bwd_tensors(q, o, lse, dq, dk, dv, delta, with_delta=True):
    """Check the forward's outputs and the backward's outputs and Δ
    workspace (allocated when None; none with with_delta=False) against
    q's shape and device."""
    B, N, H, D = q.shape
    f32, dev = torch.float32, q.device
    _need(o, q.shape, (f32, torch.bfloat16), dev, "o")
    _need(lse, (B, H, N), f32, dev, "lse")
    mk = lambda: torch.empty((B, N, H, D), dtype=f32, device=dev)
    dq = _need(mk() if dq is None else dq, q.shape, f32, dev, "dq")
    dk = _need(mk() if dk is None else dk, q.shape, f32, dev, "dk")
    dv = _need(mk() if dv is None else dv, q.shape, f32, dev, "dv")
    if not with_delta:
        return dq, dk, dv, None
    if delta is None:
        delta = torch.empty((B, H, N), dtype=f32, device=dev)
    _need(delta, (B, H, N), f32, dev, "delta")
    return dq, dk, dv, delta


def bwd(q, k, v, o, lse, dout, *, G: int, shift: int | None = None,
        boundary="wrap", valid_len: int | None = None,
        scale: float | None = None, dq=None, dk=None, dv=None, delta=None,
        doc_ids=None):
    """S²-Attn backward from the forward's o and lse.
    Returns (dq, dk, dv), float32 [B,N,H,D]."""
    B, N, H, D = _check_qkv(q, k, v, dout)
    shift = G // 2 if shift is None else shift
    valid_len = N if valid_len is None else valid_len
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    dq, dk, dv, delta = _bwd_tensors(q, o, lse, dq, dk, dv, delta)
    odt = _lib.S2A_F32 if o.dtype == torch.float32 else _lib.S2A_BF16
    lib = _lib.load()
    _lib.check(lib.s2attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), odt,
                              _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk),
                              _ptr(dv), _ptr(delta), B, N, H, D, G, shift,
                              _boundary(boundary), valid_len,
                              _docs(doc_ids, q), scale, _stream(q.device)))
    return dq, dk, dv


def bwd_noalloc(q, k, v, o, lse, dout, *, G: int, shift: int | None = None,
                boundary="wrap", valid_len: int | None = None,
                scale: float | None = None, dq=None, dk=None, dv=None,
                doc_ids=None):
    """bwd() without a delta workspace: the library keeps delta in a static
    device array (B*H*N <= S2A_NOALLOC_MAX_ROWS), so with dq, dk and dv
    given nothing is allocated.  Calls that overlap on one GPU race.
    Returns (dq, dk, dv), float32 [B,N,H,D]."""
    B, N, H, D = _check_qkv(q, k, v, dout)
    shift = G // 2 if shift is None else shift
    valid_len = N if valid_len is None else valid_len
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    dq, dk, dv, _ = _bwd_tensors(q, o, lse, dq, dk, dv, None,
                                 with_delta=False)
    odt = _lib.S2A_F32 if o.dtype == torch.float32 else _lib.S2A_BF16
    _lib.check(_lib.load().s2attn_bwd_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), odt, _ptr(lse), _ptr(dout),
        _ptr(dq), _ptr(dk), _ptr(dv), B, N, H, D, G, shift,
        _boundary(boundary), valid_len, _docs(doc_ids, q), scale,
        _stream(q.device)))
    return dq, dk, dv


def ds_workspace_bytes(B: int, N: int, H: int, D: int, *, G: int,
                       shift: int | None = None, boundary="wrap") -> int:
    """Bytes of the dS workspace that bwd_ds needs (D in {64, 128})."""
    shift = G // 2 if shift is None else shift
    out = ctypes.c_size_t(0)
    _lib.check(_lib.load().s2attn_bwd_ds_workspace(
        B, N, H, D, G, shift, _boundary(boundary), ctypes.byref(out)))
    return int(out.value)


def ds_workspace(q, *, G: int, shift: int | None = None, boundary="wrap"):
    """A device buffer for bwd_ds / bwd_dkdv_ds / bwd_dq_ds (uint8)."""
    B, N, H, D = q.shape
    n = ds_workspace_bytes(B, N, H, D, G=G, shift=shift, boundary=boundary)
    return torch.empty(max(n, 16), dtype=torch.uint8, device=q.device)


def _ds_arg(ds_ws, dev):
    if not isinstance(ds_ws, torch.Tensor) or ds_ws.dtype != torch.uint8 \
            or ds_ws.dim() != 1 or not ds_ws.is_contiguous() \
            or ds_ws.device != dev:
        raise ValueError(f"ds_ws must be a contiguous 1-D uint8 tensor on "
                         f"{dev}")
    return ds_ws.data_ptr(), ds_ws.numel()


def bwd_ds(q, k, v, o, lse, dout, *, G: int, shift: int | None = None,
           boundary="wrap", valid_len: int | None = None,
           scale: float | None = None, dq=None, dk=None, dv=None, delta=None,
           ds_ws=None):
    """The backward that stores dS in a workspace (dK/dV) and reads it for
    dQ instead of recomputing S and dP.  D in {64, 128}, no document mask.
    Returns (dq, dk, dv), float32 [B,N,H,D]."""
    B, N, H, D = _check_qkv(q, k, v, dout)
    shift = G // 2 if shift is None else shift
    valid_len = N if valid_len is None else valid_len
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    dq, dk, dv, delta = _bwd_tensors(q, o, lse, dq, dk, dv, delta)
    if ds_ws is None:
        ds_ws = ds_workspace(q, G=G, shift=shift, boundary=boundary)
    wp, wn = _ds_arg(ds_ws, q.device)
    odt = _lib.S2A_F32 if o.dtype == torch.float32 else _lib.S2A_BF16
    _lib.check(_lib.load().s2attn_bwd_ds(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), odt, _ptr(lse), _ptr(dout),
        _ptr(dq), _ptr(dk), _ptr(dv), _ptr(delta), wp, wn, B, N, H, D, G,
        shift, _boundary(boundary), valid_len, scale, _stream(q.device)))
    return dq, dk, dv


def bwd_preprocess(o, dout, delta):
    """First backward stage: delta = rowsum(dout * o)."""
    B, N, H, D = _check_qkv(dout)
    _need(o, dout.shape, (torch.float32, torch.bfloat16), dout.device, "o")
    _need(delta, (B, H, N), torch.float32, dout.device, "delta")
    odt = _lib.S2A_F32 if o.dtype == torch.float32 else _lib.S2A_BF16
    lib = _lib.load()
    _lib.check(lib.s2attn_bwd_preprocess(_ptr(o), odt, _ptr(dout),
                                         _ptr(delta), B, N, H, D,
                                         _stream(dout.device)))


def _stage_args(q, G, shift, valid_len, scale, lse=None, delta=None,
                outs=()):
    """Defaults of a stage call, after checking its statistics (lse,
    delta: float32 [B,H,N]) and its float32 [B,N,H,D] outputs."""
    B, N, H, D = q.shape
    for t, name in ((lse, "lse"), (delta, "delta")):
        if t is not None:
            _need(t, (B, H, N), torch.float32, q.device, name)
    for t, name in outs:
        _need(t, q.shape, torch.float32, q.device, name)
    shift = G // 2 if shift is None else shift
    valid_len = N if valid_len is None else valid_len
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    return B, N, H, D, G, shift, valid_len, scale


def bwd_dkdv(q, k, v, lse, delta, dout, dk, dv, *, G: int,
             shift: int | None = None, boundary="wrap",
             valid_len: int | None = None, scale: float | None = None,
             doc_ids=None):
    """dK/dV stage (needs delta from bwd_preprocess)."""
    _check_qkv(q, k, v, dout)
    B, N, H, D, G, shift, valid_len, scale = _stage_args(
        q, G, shift, valid_len, scale, lse, delta, ((dk, "dk"), (dv, "dv")))
    lib = _lib.load()
    _lib.check(lib.s2attn_bwd_dkdv(_ptr(q), _ptr(k), _ptr(v), _ptr(lse),
                                   _ptr(delta), _ptr(dout), _ptr(dk),
                                   _ptr(dv), B, N, H, D, G, shift,
                                   _boundary(boundary), valid_len,
                                   _docs(doc_ids, q), scale,
                                   _stream(q.device)))


def bwd_dq(q, k, v, lse, delta, dout, dq, *, G: int,
           shift: int | None = None, boundary="wrap",
           valid_len: int | None = None, scale: float | None = None,
           doc_ids=None):
    """dQ stage (needs delta from bwd_preprocess)."""
    _check_qkv(q, k, v, dout)
    B, N, H, D, G, shift, valid_len, scale = _stage_args(
        q, G, shift, valid_len, scale, lse, delta, ((dq, "dq"),))
    lib = _lib.load()
    _lib.check(lib.s2attn_bwd_dq(_ptr(q), _ptr(k), _ptr(v), _ptr(lse),
                                 _ptr(delta), _ptr(dout), _ptr(dq), B, N, H,
                                 D, G, shift, _boundary(boundary), valid_len,
                                 _docs(doc_ids, q), scale, _stream(q.device)))


def bwd_dkdv_ds(q, k, v, lse, delta, dout, dk, dv, ds_ws, *, G: int,
                shift: int | None = None, boundary="wrap",
                valid_len: int | None = None, scale: float | None = None):
    """The dK/dV stage of bwd_ds (fills ds_ws); for timing one kernel."""
    _check_qkv(q, k, v, dout)
    B, N, H, D, G, shift, valid_len, scale = _stage_args(
        q, G, shift, valid_len, scale, lse, delta, ((dk, "dk"), (dv, "dv")))
    wp, wn = _ds_arg(ds_ws, q.device)
    _lib.check(_lib.load().s2attn_bwd_dkdv_ds(
        _ptr(q), _ptr(k), _ptr(v), _ptr(lse), _ptr(delta), _ptr(dout),
        _ptr(dk), _ptr(dv), wp, wn, B, N, H, D, G, shift, _boundary(boundary),
        valid_len, scale, _stream(q.device)))


def bwd_dq_ds(k, ds_ws, dq, *, G: int, shift: int | None = None,
              boundary="wrap", valid_len: int | None = None,
              scale: float | None = None):
    """The dQ stage of bwd_ds: dq from the dS that bwd_dkdv_ds stored."""
    _check_qkv(k)
    B, N, H, D, G, shift, valid_len, scale = _stage_args(
        k, G, shift, valid_len, scale, outs=((dq, "dq"),))
    wp, wn = _ds_arg(ds_ws, k.device)
    _lib.check(_lib.load().s2attn_bwd_dq_ds(
        _ptr(k), wp, wn, _ptr(dq), B, N, H, D, G, shift, _boundary(boundary),
        valid_len, scale, _stream(k.device)))


def shard_halo(N: int, row0: int, T: int, *, G: int, shift: int | None = None,
               boundary="wrap", valid_len: int | None = None):
    """Halo of the slice [row0, row0 + T) of a sequence of padded length N:
    (left_first, left_rows, wrap_rows).  The left halo is global rows
    [left_first, left_first + left_rows), stored right before the slice's
    row 0; the wrap halo is rows [0, wrap_rows), stored 2s rows before it.
    Host arithmetic of the library; nothing runs on the device."""
    import ctypes
    shift = G // 2 if shift is None else shift
    valid_len = N if valid_len is None else valid_len
    out = [ctypes.c_int(0) for _ in range(3)]
    lib = _lib.load()
    _lib.check(lib.s2attn_shard_halo(N, row0, T, G, shift,
                                     _boundary(boundary), valid_len,
                                     *(ctypes.byref(o) for o in out)))
    return tuple(o.value for o in out)


def _shard_args(q, k_ext, v_ext, N, row0, G, shift, boundary, valid_len,
                scale, doc_ext):
    if q.dim() != 3:
        raise ValueError("q must be [T, H, D] (one sequence)")
    T, H, D = q.shape
    for t in (q, k_ext, v_ext):
        if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous():
            raise ValueError("q, k, v must be contiguous bfloat16 GPU tensors")
    if k_ext.shape != v_ext.shape or k_ext.dim() != 3 \
            or tuple(k_ext.shape[1:]) != (H, D) or k_ext.shape[0] < T:
        raise ValueError("k, v must be [R + T, H, D]: R halo rows, then the "
                         "slice's T rows")
    shift = G // 2 if shift is None else shift
    valid_len = N if valid_len is None else valid_len
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    R = k_ext.shape[0] - T
    _, left_rows, wrap_rows = shard_halo(N, row0, T, G=G, shift=shift,
                                         boundary=boundary,
                                         valid_len=valid_len)
    s = shift if N // G > 1 else 0
    need = 2 * s if wrap_rows else left_rows
    if R < need:
        raise ValueError(f"k, v hold {R} halo rows; this slice needs {need}")
    doc = None
    if doc_ext is not None:
        if doc_ext.dtype != torch.int32 or tuple(doc_ext.shape) != (R + T,) \
                or not doc_ext.is_contiguous() or doc_ext.device != q.device:
            raise ValueError("doc_ids must be a contiguous int32 [R + T] "
                             "tensor in the layout of k")
        doc = doc_ext.data_ptr() + 4 * R
    off = R * H * D * 2  # bytes to the slice's row 0
    return (T, H, D, shift, valid_len, scale, R, k_ext.data_ptr() + off,
            v_ext.data_ptr() + off, doc)


def _out(t, shape, dtype, dev, name, zero=False):
    if t is None:
        return (torch.zeros if zero else torch.empty)(shape, dtype=dtype,
                                                      device=dev)
    return _need(t, shape, dtype, dev, name)


def fwd_shard(q, k_ext, v_ext, *, N: int, row0: int, G: int,
              shift: int | None = None, boundary="wrap",
              valid_len: int | None = None, scale: float | None = None,
              out_dtype=torch.float32, doc_ext=None, o=None, lse=None):
    """Forward of the slice [row0, row0 + T) of a sequence of padded length
    N (sequence parallelism).  q [T, H, D]; k_ext, v_ext [R + T, H, D]
    with the slice's rows last and the halo (see shard_halo) in the R rows
    before them; doc_ext: optional int32 [R + T] in the same layout.
    Returns (o [T, H, D], lse [H, T] float32)."""
    T, H, D, shift, valid_len, scale, R, kp, vp, doc = _shard_args(
        q, k_ext, v_ext, N, row0, G, shift, boundary, valid_len, scale,
        doc_ext)
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("out_dtype must be float32 or bfloat16")
    o = _out(o, (T, H, D), out_dtype, q.device, "o")
    lse = _out(lse, (H, T), torch.float32, q.device, "lse")
    odt = _lib.S2A_F32 if out_dtype == torch.float32 else _lib.S2A_BF16
    lib = _lib.load()
    _lib.check(lib.s2attn_fwd_shard(_ptr(q), kp, vp, _ptr(o), odt, _ptr(lse),
                                    N, row0, T, H, D, G, shift,
                                    _boundary(boundary), valid_len, doc,
                                    scale, _stream(q.device)))
    return o, lse


def bwd_shard(q, k_ext, v_ext, o, lse, dout, *, N: int, row0: int, G: int,
              shift: int | None = None, boundary="wrap",
              valid_len: int | None = None, scale: float | None = None,
              doc_ext=None, dq=None, dk=None, dv=None, delta=None):
    """Backward of a slice from its forward's o and lse.  Returns (dq
    [T, H, D], dk_ext, dv_ext [R + T, H, D]), float32: rows R.. are the
    slice's keys, and the halo rows of the shifted heads hold the partial
    gradients of the neighbours' keys.  Rows the kernels do not write keep
    what dk, dv held (zeros when they are allocated here)."""
    T, H, D, shift, valid_len, scale, R, kp, vp, doc = _shard_args(
        q, k_ext, v_ext, N, row0, G, shift, boundary, valid_len, scale,
        doc_ext)
    _need(dout, q.shape, torch.bfloat16, q.device, "dout")
    _need(o, q.shape, (torch.float32, torch.bfloat16), q.device, "o")
    _need(lse, (H, T), torch.float32, q.device, "lse")
    f32, dev = torch.float32, q.device
    dq = _out(dq, (T, H, D), f32, dev, "dq")
    dk = _out(dk, (R + T, H, D), f32, dev, "dk", zero=True)
    dv = _out(dv, (R + T, H, D), f32, dev, "dv", zero=True)
    delta = _out(delta, (H, T), f32, dev, "delta")
    off = R * H * D * 4
    odt = _lib.S2A_F32 if o.dtype == torch.float32 else _lib.S2A_BF16
    lib = _lib.load()
    _lib.check(lib.s2attn_bwd_shard(_ptr(q), kp, vp, _ptr(o), odt, _ptr(lse),
                                    _ptr(dout), _ptr(dq), dk.data_ptr() + off,
                                    dv.data_ptr() + off, _ptr(delta), N,
                                    row0, T, H, D, G, shift,
                                    _boundary(boundary), valid_len, doc,
                                    scale, _stream(q.device)))
    return dq, dk, dv


PAIRINGS = {"half": _lib.S2A_ROPE_HALF, "interleaved": _lib.S2A_ROPE_INTERLEAVED,
            _lib.S2A_ROPE_HALF: _lib.S2A_ROPE_HALF,
            _lib.S2A_ROPE_INTERLEAVED: _lib.S2A_ROPE_INTERLEAVED}


def _rope_args(x, pos_ids, pairing):
    if x.dim() != 4 or not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous [B, N, H, D] GPU tensor")
    B, N, H, D = x.shape
    pp = None
    if pos_ids is not None:
        if pos_ids.dtype != torch.int32 or tuple(pos_ids.shape) != (B, N) \
                or not pos_ids.is_contiguous() or pos_ids.device != x.device:
            raise ValueError("pos_ids must be a contiguous int32 [B, N] "
                             "tensor on the device of x")
        pp = pos_ids.data_ptr()
    try:
        pr = PAIRINGS[pairing]
    except KeyError:
        raise ValueError(f"pairing must be 'half' or 'interleaved', got "
                         f"{pairing!r}")
    return B, N, H, D, pp, pr


def rope(x, *, base: float = 10000.0, pos_scale: float = 1.0, pos_ids=None,
         pairing="half", out=None):
    """Rotary position embedding of bf16 [B,N,H,D] at global positions
    (pos_ids int32 [B,N], default 0..N-1), scaled by pos_scale (linear
    position interpolation).  out may be x (in place)."""
    if x.dtype != torch.bfloat16:
        raise ValueError("x must be bfloat16")
    B, N, H, D, pp, pr = _rope_args(x, pos_ids, pairing)
    out = torch.empty_like(x) if out is None else out
    _need(out, x.shape, torch.bfloat16, x.device, "out")
    lib = _lib.load()
    _lib.check(lib.s2attn_rope(_ptr(x), _ptr(out), B, N, H, D, pp, base,
                               pos_scale, pr, _stream(x.device)))
    return out


def rope_bwd(gy, *, base: float = 10000.0, pos_scale: float = 1.0,
             pos_ids=None, pairing="half", out=None):
    """Gradient of rope(): R^T applied to float32 [B,N,H,D] gradients.
    out may be gy (in place)."""
    if gy.dtype != torch.float32:
        raise ValueError("gy must be float32")
    B, N, H, D, pp, pr = _rope_args(gy, pos_ids, pairing)
    out = torch.empty_like(gy) if out is None else out
    _need(out, gy.shape, torch.float32, gy.device, "out")
    lib = _lib.load()
    _lib.check(lib.s2attn_rope_bwd(_ptr(gy), _ptr(out), B, N, H, D, pp, base,
                                   pos_scale, pr, _stream(gy.device)))
    return out


def group_map(N: int, G: int, *, shift: int | None = None, boundary="wrap",
              valid_len: int | None = None, device="cuda"):
    """Group index maps (gid, slot, src), each int32 [2, N] on the device."""
    shift = G // 2 if shift is None else shift
    valid_len = N if valid_len is None else valid_len
    outs = [torch.empty((2, N), dtype=torch.int32, device=device)
            for _ in range(3)]
    lib = _lib.load()
    _lib.check(lib.s2attn_group_map(N, G, shift, _boundary(boundary),
                                    valid_len, *(_ptr(t) for t in outs),
                                    _stream(outs[0].device)))
    return tuple(outs)


BACKWARDS = ("auto", "stored_ds", "recompute")


def _backward(q, k, v, o, lse, do, G, shift, boundary, valid_len, scale,
              doc_ids, which):
    """The backward the autograd op runs.  "stored_ds" keeps dS in a
    workspace (2 bytes per allowed pair, allocated through torch's caching
    allocator) and forms dQ from it; it covers D in {64, 128} without a
    document mask and is the faster one at every measured workload.
    "recompute" forms dQ by recomputing S and dP and needs only a B*H*N
    workspace.  "auto" takes stored_ds where it applies and its workspace
    can be allocated, else recompute."""
    D = q.shape[3]
    stored_ok = D in (64, 128) and doc_ids is None
    if which == "stored_ds" and not stored_ok:
        raise ValueError("the stored-dS backward needs D in {64, 128} and no "
                         "document mask")
    kw = dict(G=G, shift=shift, boundary=boundary, valid_len=valid_len,
              scale=scale)
    if which != "recompute" and stored_ok:
        try:
            ws = ds_workspace(q, G=G, shift=shift, boundary=boundary)
        except torch.cuda.OutOfMemoryError:
            if which == "stored_ds":
                raise
            ws = None
        if ws is not None:
            return bwd_ds(q, k, v, o, lse, do, ds_ws=ws, **kw)
    return bwd(q, k, v, o, lse, do, doc_ids=doc_ids, **kw)


class S2AttnFunction(torch.autograd.Function):
    """Autograd wrapper: forward and backward both run in the library.
    With rope (a dict of rope() keywords) q and k are the unrotated
    projections: they are rotated at their global positions first, and the
    gradients are rotated back.  backward_kind picks the backward (see
    _backward)."""

    @staticmethod
    def forward(ctx, q, k, v, G, shift, boundary, valid_len, scale,
                doc_ids=None, rope_cfg=None, backward_kind="auto"):
        if backward_kind not in BACKWARDS:
            raise ValueError(f"backward must be one of {BACKWARDS}")
        if rope_cfg is not None:
            q = rope(q, **rope_cfg)
            k = rope(k, **rope_cfg)
        o, lse = fwd(q, k, v, G=G, shift=shift, boundary=boundary,
                     valid_len=valid_len, scale=scale, doc_ids=doc_ids)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.cfg = (G, shift, boundary, valid_len, scale, doc_ids, rope_cfg,
                   backward_kind)
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse = ctx.saved_tensors
        (G, shift, boundary, valid_len, scale, doc_ids, rope_cfg,
         which) = ctx.cfg
        dq, dk, dv = _backward(q, k, v, o, lse,
                               do.to(torch.bfloat16).contiguous(), G, shift,
                               boundary, valid_len, scale, doc_ids, which)
        if rope_cfg is not None:
            rope_bwd(dq, out=dq, **rope_cfg)
            rope_bwd(dk, out=dk, **rope_cfg)
        return (dq.to(q.dtype), dk.to(k.dtype), dv.to(v.dtype),
                None, None, None, None, None, None, None, None)


def s2_attention(q, k, v, G, shift=None, boundary="wrap", valid_len=None,
                 scale=None, doc_ids=None, rope_cfg=None, backward="auto"):
    """Differentiable S²-Attn (float32 output).  rope_cfg: None, or a dict
    of rope() keywords (base, pos_scale, pos_ids, pairing) to rotate q and
    k at their global positions inside the op.  backward: "auto" (the
    stored-dS backward where it applies, see _backward), "stored_ds" or
    "recompute"."""
    return S2AttnFunction.apply(q, k, v, G, shift, boundary, valid_len, scale,
                                doc_ids, rope_cfg, backward)
