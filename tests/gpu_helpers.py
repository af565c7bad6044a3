"""Shared helpers of the GPU parity tests: move the seeded bf16 inputs to
the device, widen the same bits to float64 for the oracle, and compare."""
import math
import sys

import numpy as np
import torch

import synthetic as syn

ATOL_MAX = 1e-2     # max |gpu - oracle| for o, dq, dk, dv
ATOL_MEAN = 1e-3    # mean |gpu - oracle|
LSE_TOL = 1e-3      # max |gpu - oracle| for lse over valid rows


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(bits: np.ndarray) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).cuda()


def heads_f64(bits: np.ndarray, heads):
    """float64 copy of the selected heads, shape [B, N, len(heads), D]."""
    return syn.bf16_bits_to_f64(bits[:, :, list(heads), :])


def compare(name, got, want, valid_rows=None, atol_max=ATOL_MAX,
            atol_mean=ATOL_MEAN):
    """got/want [B, N, h, D]; rows >= valid length must be exactly zero."""
    got = np.asarray(got, dtype=np.float64)
    err = np.abs(got - want)
    mx, mean = float(err.max()), float(err.mean())
    where = np.unravel_index(int(err.argmax()), err.shape)
    say(f"  {name}: max|d|={mx:.3e} at {tuple(int(i) for i in where)} "
        f"mean|d|={mean:.3e}")
    assert mx <= atol_max, f"{name} max abs diff {mx} > {atol_max}"
    assert mean <= atol_mean, f"{name} mean abs diff {mean} > {atol_mean}"
    if valid_rows is not None:
        assert np.all(got[:, valid_rows:] == 0), f"{name}: padded rows not zero"


def compare_lse(got, want, L):
    """got/want [B, h, N]."""
    got = np.asarray(got, dtype=np.float64)
    fin = np.isfinite(want)
    assert np.array_equal(fin[..., :L], np.ones_like(fin[..., :L]))
    err = float(np.abs(got[..., :L] - want[..., :L]).max())
    say(f"  lse: max|d|={err:.3e}")
    assert err <= LSE_TOL
    if L < got.shape[-1]:
        assert np.all(np.isneginf(got[..., L:])), "padded lse rows not -inf"


def scale_for(D):
    return 1.0 / math.sqrt(D)
