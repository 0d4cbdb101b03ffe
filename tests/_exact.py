"""Exact reference helpers for pinning the oracle (CPU only, tiny inputs).

They take their values from torch's own conversions (FP8 -> float32 and
BF16 -> float32 decode of every bit pattern), and do all arithmetic in
``fractions.Fraction``; nothing here reuses the oracle's tables or code.
"""
from __future__ import annotations

import bisect
import math
from fractions import Fraction
from functools import lru_cache

import numpy as np
import torch


@lru_cache(maxsize=None)
def fp8_values(fmt: int):
    """Python floats of all 256 codes via torch's float8 -> float32 conversion."""
    dt = torch.float8_e4m3fn if fmt == 0 else torch.float8_e5m2
    return tuple(float(v) for v in torch.arange(256, dtype=torch.uint8).view(dt).float().tolist())


@lru_cache(maxsize=None)
def _bf16_table():
    """Sorted finite non-negative BF16 values with their bit patterns."""
    bits = torch.arange(0x8000, dtype=torch.int32).to(torch.int16)
    vals = bits.view(torch.bfloat16).float().double().numpy()
    pairs = [(Fraction(float(v)), int(b)) for b, v in zip(range(0x8000), vals) if math.isfinite(v)]
    pairs.sort()
    return [p[0] for p in pairs], [p[1] for p in pairs]


def bf16_nearest_even(x) -> int:
    """BF16 bits nearest to x (a Fraction or float), ties to the even pattern,
    overflow past the largest finite value (by at least half a step) to inf.
    Found by search over every finite BF16 value."""
    if isinstance(x, float):
        if math.isnan(x):
            return 0x7FC0
        if math.isinf(x):
            return 0x7F80 if x > 0 else 0xFF80
        x = Fraction(x)
    sign = 0x8000 if x < 0 else 0
    a = -x if x < 0 else x
    vals, bits = _bf16_table()
    top = vals[-1]
    step = top - vals[-2]
    if a >= top + step / 2:
        if a == top + step / 2 and (bits[-1] & 1) == 0:
            return sign | bits[-1]
        return sign | 0x7F80
    i = bisect.bisect_left(vals, a)
    if i < len(vals) and vals[i] == a:
        return sign | bits[i]
    lo, hi = vals[i - 1], vals[i]
    if a - lo < hi - a:
        pick = bits[i - 1]
    elif a - lo > hi - a:
        pick = bits[i]
    else:
        pick = bits[i - 1] if (bits[i - 1] & 1) == 0 else bits[i]
    if a == 0:
        return sign
    return sign | pick


def exact_gemm(A, B, a_fmt, b_fmt, sa=1.0, sb=1.0):
    """Exact D bits for tiny A [M, K], B [N, K] (uint8 codes).  Non-finite
    inputs follow IEEE float semantics in Python floats."""
    va, vb = fp8_values(a_fmt), fp8_values(b_fmt)
    M, K = A.shape
    N = B.shape[0]
    D = np.zeros((M, N), dtype=np.uint16)
    sc = Fraction(float(np.float32(sa))) * Fraction(float(np.float32(sb)))
    for i in range(M):
        for j in range(N):
            fa = [va[c] for c in A[i]]
            fb = [vb[c] for c in B[j]]
            if all(math.isfinite(p) for p in fa + fb):
                s = sum((Fraction(p) * Fraction(q) for p, q in zip(fa, fb)), Fraction(0))
                D[i, j] = bf16_nearest_even(s * sc)
            else:
                s = 0.0
                for p, q in zip(fa, fb):
                    s += p * q
                D[i, j] = bf16_nearest_even(s * float(sc)) if not math.isfinite(s) else bf16_nearest_even(Fraction(s) * sc)
    return D
