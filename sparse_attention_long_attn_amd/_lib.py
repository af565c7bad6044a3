"""ctypes view of libs2attn.so (the C ABI declared in include/s2attn.h).

Loading needs only the ROCm runtime library, not a GPU, so the exported
symbols and the argument checks (which fail before anything touches the
device) can be exercised on a CPU-only host.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libs2attn.so")

# rows (B*H*N) of the delta array s2attn_bwd_noalloc keeps on the device
S2A_NOALLOC_MAX_ROWS = 1 << 22

S2A_OK, S2A_EINVAL, S2A_EUNSUPPORTED, S2A_EHIP = 0, 1, 2, 3
S2A_WRAP, S2A_SPLIT, S2A_CYCLIC = 0, 1, 2
S2A_BF16, S2A_F32 = 0, 1
S2A_ROPE_HALF, S2A_ROPE_INTERLEAVED = 0, 1

EXPORTS = ("s2attn_fwd", "s2attn_bwd", "s2attn_bwd_preprocess",
           "s2attn_bwd_dkdv", "s2attn_bwd_dq", "s2attn_group_map",
           "s2attn_rope", "s2attn_rope_bwd", "s2attn_shard_halo",
           "s2attn_fwd_shard", "s2attn_bwd_shard",
           "s2attn_bwd_ds_workspace", "s2attn_bwd_ds", "s2attn_bwd_dkdv_ds",
           "s2attn_bwd_dq_ds", "s2attn_bwd_noalloc",
           "s2attn_strerror", "s2attn_last_error", "s2attn_version")

_lib = None


class S2AttnError(RuntimeError):
    """A HIP launch failure reported by the library."""


def load() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with "
            "`python -m sparse_attention_long_attn_amd.build` (there is no "
            "fallback implementation)")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    # ... boundary, valid_len, doc_ids, scale, stream
    lib.s2attn_fwd.argtypes = [P, P, P, P, I, P, I, I, I, I, I, I, I, I, P, F,
                               P]
    lib.s2attn_fwd.restype = I
    lib.s2attn_bwd.argtypes = [P, P, P, P, I, P, P, P, P, P, P,
                               I, I, I, I, I, I, I, I, P, F, P]
    lib.s2attn_bwd.restype = I
    lib.s2attn_bwd_noalloc.argtypes = [P, P, P, P, I, P, P, P, P, P,
                                       I, I, I, I, I, I, I, I, P, F, P]
    lib.s2attn_bwd_noalloc.restype = I
    lib.s2attn_bwd_preprocess.argtypes = [P, I, P, P, I, I, I, I, P]
    lib.s2attn_bwd_preprocess.restype = I
    lib.s2attn_bwd_dkdv.argtypes = [P, P, P, P, P, P, P, P,
                                    I, I, I, I, I, I, I, I, P, F, P]
    lib.s2attn_bwd_dkdv.restype = I
    lib.s2attn_bwd_dq.argtypes = [P, P, P, P, P, P, P,
                                  I, I, I, I, I, I, I, I, P, F, P]
    lib.s2attn_bwd_dq.restype = I
    lib.s2attn_group_map.argtypes = [I, I, I, I, I, P, P, P, P]
    lib.s2attn_group_map.restype = I
    # N, row0, T, G, shift, boundary, valid_len, 3 int* outputs
    lib.s2attn_shard_halo.argtypes = [I, I, I, I, I, I, I, P, P, P]
    lib.s2attn_shard_halo.restype = I
    # q, k, v, o, o_dtype, lse, N, row0, T, H, D, G, shift, boundary,
    # valid_len, doc_ids, scale, stream
    lib.s2attn_fwd_shard.argtypes = [P, P, P, P, I, P, I, I, I, I, I, I, I,
                                     I, I, P, F, P]
    lib.s2attn_fwd_shard.restype = I
    lib.s2attn_bwd_shard.argtypes = [P, P, P, P, I, P, P, P, P, P, P,
                                     I, I, I, I, I, I, I, I, I, P, F, P]
    lib.s2attn_bwd_shard.restype = I
    Z = ctypes.c_size_t
    # B, N, H, D, G, shift, boundary, bytes*
    lib.s2attn_bwd_ds_workspace.argtypes = [I, I, I, I, I, I, I,
                                            ctypes.POINTER(Z)]
    lib.s2attn_bwd_ds_workspace.restype = I
    lib.s2attn_bwd_ds.argtypes = [P, P, P, P, I, P, P, P, P, P, P, P, Z,
                                  I, I, I, I, I, I, I, I, F, P]
    lib.s2attn_bwd_ds.restype = I
    lib.s2attn_bwd_dkdv_ds.argtypes = [P, P, P, P, P, P, P, P, P, Z,
                                       I, I, I, I, I, I, I, I, F, P]
    lib.s2attn_bwd_dkdv_ds.restype = I
    lib.s2attn_bwd_dq_ds.argtypes = [P, P, Z, P, I, I, I, I, I, I, I, I, F, P]
    lib.s2attn_bwd_dq_ds.restype = I
    # x, y, B, N, H, D, pos_ids, base, pos_scale, pairing, stream
    for fn in (lib.s2attn_rope, lib.s2attn_rope_bwd):
        fn.argtypes = [P, P, I, I, I, I, P, F, F, I, P]
        fn.restype = I
    lib.s2attn_strerror.argtypes = [I]
    lib.s2attn_strerror.restype = ctypes.c_char_p
    lib.s2attn_last_error.argtypes = []
    lib.s2attn_last_error.restype = ctypes.c_char_p
    lib.s2attn_version.argtypes = []
    lib.s2attn_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


def check(status: int) -> None:
    """Raise for a non-OK status: ValueError for bad arguments or an
    unsupported width, S2AttnError for a HIP failure."""
    if status == S2A_OK:
        return
    lib = load()
    msg = (f"{lib.s2attn_strerror(status).decode()}: "
           f"{lib.s2attn_last_error().decode()}")
    if status in (S2A_EINVAL, S2A_EUNSUPPORTED):
        raise ValueError(msg)
    raise S2AttnError(msg)
