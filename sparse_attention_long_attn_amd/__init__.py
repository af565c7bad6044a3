"""MI355X (gfx950) shifted sparse attention (S²-Attn) engine.

The computation lives in libs2attn.so (hand-written HIP kernels behind the
C ABI of include/s2attn.h).  This package only builds that library and
marshals torch tensors into its calls.
"""
from . import _lib, work  # noqa: F401
from ._lib import S2A_WRAP, S2A_SPLIT, S2AttnError, load  # noqa: F401
from .ops import (fwd, bwd, bwd_preprocess, bwd_dkdv, bwd_dq,  # noqa: F401
                  group_map, rope, rope_bwd, s2_attention, S2AttnFunction,
                  shard_halo, fwd_shard, bwd_shard, ds_workspace_bytes,
                  ds_workspace, bwd_ds, bwd_dkdv_ds, bwd_dq_ds,
                  bwd_noalloc)

__all__ = ["fwd", "bwd", "bwd_preprocess", "bwd_dkdv",
           "bwd_dq", "group_map", "rope", "rope_bwd", "s2_attention",
           "S2AttnFunction", "shard_halo", "fwd_shard", "bwd_shard",
           "ds_workspace_bytes", "ds_workspace", "bwd_ds", "bwd_dkdv_ds",
           "bwd_dq_ds", "bwd_noalloc",
           "S2A_WRAP", "S2A_SPLIT", "S2AttnError", "load", "work"]
