"""Pins for the oracle's per-channel form: D = bf16(sa[m] sb[n] A[m].B[n] + bias[n]).

Compared with exact rational arithmetic on torch's FP8 decode (brute force on
tiny inputs), the per-tensor oracle (pinned separately) where the vectors are
uniform, a closed form (all-zero weights leave exactly the rounded bias), and
exact linearity in one row's or one channel's scale.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from tests._exact import bf16_nearest_even, fp8_values

E4M3, E5M2 = oracle.E4M3, oracle.E5M2


def _finite(rng, shape):
    c = rng.integers(0, 256, size=shape).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x38
    return c


@pytest.mark.parametrize("a_fmt,b_fmt", [(E4M3, E4M3), (E5M2, E4M3)])
def test_matches_exact_rational(a_fmt, b_fmt):
    rng = np.random.default_rng(11 + a_fmt)
    M, N, K = 4, 6, 48
    A = _finite(rng, (M, K))
    B = _finite(rng, (N, K))
    if a_fmt == E5M2:
        A[(A & 0x7C) == 0x7C] = 0x3C
    sa = rng.uniform(0.1, 3, M).astype(np.float32)
    sb = rng.uniform(-2, 2, N).astype(np.float32)
    bias = rng.normal(0, 50, N).astype(np.float32)
    D, R, S = oracle.gemm_nt_channelwise(A, B, sa, sb, bias, a_fmt, b_fmt)
    va, vb = fp8_values(a_fmt), fp8_values(b_fmt)
    for m in range(M):
        for n in range(N):
            acc = sum(Fraction(va[A[m, k]]) * Fraction(vb[B[n, k]]) for k in range(K))
            ex = Fraction(float(sa[m])) * Fraction(float(sb[n])) * acc + Fraction(float(bias[n]))
            assert D[m, n] == bf16_nearest_even(ex), (m, n)
            assert abs(Fraction(R[m, n]) - ex) <= (abs(ex) + abs(Fraction(float(bias[n])))) * Fraction(1, 2 ** 50)


def test_uniform_vectors_equal_per_tensor():
    rng = np.random.default_rng(12)
    A = _finite(rng, (9, 64))
    B = _finite(rng, (7, 64))
    D, R, S = oracle.gemm_nt_channelwise(A, B, np.full(9, 0.75, np.float32), np.full(7, 1.5, np.float32), None)
    D1, R1, S1, _ = oracle.gemm_nt(A, B, sa=0.75, sb=1.5)
    assert np.array_equal(D, D1) and np.array_equal(R, R1)
    np.testing.assert_allclose(S, S1 * 0.75 * 1.5, rtol=1e-15)


def test_zero_weights_give_the_rounded_bias():
    rng = np.random.default_rng(13)
    A = _finite(rng, (5, 32))
    B = np.zeros((300, 32), np.uint8)
    bias = rng.normal(0, 1e3, 300).astype(np.float32)
    D, R, _ = oracle.gemm_nt_channelwise(A, B, rng.uniform(1, 2, 5).astype(np.float32), None, bias)
    want = np.array([bf16_nearest_even(float(b)) for b in bias], np.uint16)
    assert all(np.array_equal(D[m], want) for m in range(5))


def test_missing_vectors_are_ones_and_zeros():
    rng = np.random.default_rng(14)
    A = _finite(rng, (3, 32))
    B = _finite(rng, (4, 32))
    D0, R0, _ = oracle.gemm_nt_channelwise(A, B, None, None, None)
    D1, R1, _ = oracle.gemm_nt_channelwise(A, B, np.ones(3, np.float32), np.ones(4, np.float32), np.zeros(4, np.float32))
    assert np.array_equal(D0, D1) and np.array_equal(R0, R1)


def test_row_and_channel_scales_are_exactly_linear():
    rng = np.random.default_rng(15)
    A = _finite(rng, (6, 64))
    B = _finite(rng, (5, 64))
    sa = rng.uniform(0.5, 1, 6).astype(np.float32)
    sb = rng.uniform(0.5, 1, 5).astype(np.float32)
    _, R, _ = oracle.gemm_nt_channelwise(A, B, sa, sb, None)
    sa2 = sa.copy(); sa2[2] *= 4
    sb2 = sb.copy(); sb2[3] *= 0.5
    _, R2, _ = oracle.gemm_nt_channelwise(A, B, sa2, sb2, None)
    want = R.copy(); want[2, :] *= 4; want[:, 3] *= 0.5
    assert np.array_equal(R2, want)
