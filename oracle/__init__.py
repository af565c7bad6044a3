"""Float64 CPU oracle for shifted sparse attention (S²-Attn).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, links or
runs this package: only the tests, ``__graft_entry__.smoke()`` and the
bench's CPU-baseline leg do.  It shares no code with the HIP library.

It is a plain, slow, dense evaluation of what the method computes, written
from the definitions on the page "4.1.2 · LongLoRA: 用S²-Attn完成长上下文微调"
(PaperTrace) and the study notes "精读笔记：LongLoRA" (§3.2), in float64:

* ``group_maps_a`` / ``adjacency_block``  -- the index definitions
  (§1 "S²-Attn的计算图", the group functions b(i), b'(i) and the visible
  sets N_0(i), N_1(i); §2.2, mask equation M_h), derivation A;
* ``group_maps_b`` / ``forward_segments`` / ``backward_segments`` -- the
  shift -> reshape -> in-group causal attention -> inverse shift route of
  §1 ("Reshape如何复用普通kernel"), derivation B, written independently;
* ``forward`` / ``backward`` -- dense masked softmax attention over the
  derivation-A adjacency (§3, equation for o_i^s and the gradient
  equation for dL/dz_j);
* ``rope`` -- rotary position embedding at global positions with linear
  position interpolation (§3.1, the rotation R(m, w); §1.1 on position IDs).

Every function is pinned by tests against things other than itself (worked
examples printed on the pages, closed-form pair counts, G=N reducing to
textbook causal attention brute-forced in Python loops, a library SDPA
routine on unpadded segments, central finite differences, invariants).
"""
from .s2attn_oracle import (  # noqa: F401
    WRAP, SPLIT, CYCLIC, OracleError, effective_shift, validate, group_maps_a,
    group_maps_b, adjacency_block, adjacency_dense, allowed_pairs, forward,
    backward, forward_segments, backward_segments, segments,
)
from .rope import HALF, INTERLEAVED, frequencies, rope  # noqa: F401
