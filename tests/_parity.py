"""Element-wise comparison of the GPU output with the oracle.

The acceptance bound for every valid element d (BF16 from the GPU) against the
oracle's FP64 value r (scaled, before BF16 rounding) and S = sum_k |a_ik b_jk|:

    |d - r| <= 2^-8 |r| + 1e-5 |sa * sb| S

with NaN matching NaN and +-inf matching the same-signed infinity.  The
2^-8 |r| term covers one BF16 rounding (half an ulp is at most 2^-8 |r|); the
second term covers FP32 accumulation of K products in blocks of 64/128 plus
the FP32 scale multiply, which is far below 1e-5 S for K <= 14336.
"""
from __future__ import annotations

import numpy as np
import torch


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).double().numpy()


def gpu_bits(t: torch.Tensor) -> np.ndarray:
    """Host copy of a bfloat16 tensor as uint16 bit patterns."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def violations(d_bits, r, s, scale_abs):
    """Boolean mask of elements outside the bound (shapes broadcast)."""
    d = bf16_bits_to_f64(d_bits)
    r = np.asarray(r, dtype=np.float64)
    s = np.asarray(s, dtype=np.float64)
    scale_abs = np.asarray(scale_abs, dtype=np.float64)
    bad = np.zeros(np.broadcast(d, r).shape, dtype=bool)
    nan_r, nan_d = np.isnan(r), np.isnan(d)
    bad |= nan_r != nan_d
    inf_r, inf_d = np.isinf(r), np.isinf(d)
    both_inf = inf_r & inf_d
    bad |= (inf_r != inf_d) & ~nan_r & ~nan_d
    bad |= both_inf & (np.sign(r) != np.sign(d))
    fin = np.isfinite(r) & np.isfinite(d)
    with np.errstate(invalid="ignore", over="ignore"):
        tol = 2.0 ** -8 * np.abs(r) + 1e-5 * scale_abs * s
        bad |= fin & (np.abs(d - r) > tol)
    return bad


def assert_within_bound(d_bits, r, s, scale_abs, ref_bits=None, what=""):
    bad = violations(d_bits, r, s, scale_abs)
    n = int(bad.sum())
    if n:
        idx = np.argwhere(bad)[:8]
        d = bf16_bits_to_f64(d_bits)
        rows = []
        for ix in idx:
            t = tuple(ix)
            rows.append(f"{t}: gpu={d[t]!r} oracle={np.asarray(r)[t]!r} S={np.asarray(s)[t]!r}")
        raise AssertionError(f"{what}: {n} of {bad.size} elements outside the bound; first: " + "; ".join(rows))
    if ref_bits is not None:
        same = np.asarray(d_bits) == np.asarray(ref_bits)
        return float(same.mean()) if same.size else 1.0
    return None
