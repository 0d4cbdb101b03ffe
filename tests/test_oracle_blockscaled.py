"""Pins for the oracle's block-scaled dense GEMM (power-of-two UE8M0 scales per
128-element K block: per row of A, per 128 rows of B).

Each check compares the oracle with something other than itself: exact
rational arithmetic on torch's FP8 decode with a BF16 search (brute force on
tiny inputs), an invariance that holds only if every scale is applied to the
right rows and K block, the per-tensor oracle (pinned separately) where the
scales are uniform, and NaN propagation.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from tests._exact import bf16_nearest_even, fp8_values

E4M3, E5M2 = oracle.E4M3, oracle.E5M2


def _codes(rng, fmt, shape, lo_exp=1, hi_exp=13):
    """Random finite normal codes whose value doubles exactly by adding 1 to the
    exponent field (E4M3: fields 1..13; E5M2: fields 1..29)."""
    mbits = 3 if fmt == E4M3 else 2
    if fmt == E5M2:
        hi_exp = 29
    e = rng.integers(lo_exp, hi_exp + 1, size=shape)
    m = rng.integers(0, 1 << mbits, size=shape)
    s = rng.integers(0, 2, size=shape)
    return ((s << 7) | (e << mbits) | m).astype(np.uint8)


def _scales(rng, shape, lo=122, hi=132):
    return rng.integers(lo, hi + 1, size=shape).astype(np.uint8)


def _exact_element(A, B, sa, sb, m, n, a_fmt, b_fmt):
    va, vb = fp8_values(a_fmt), fp8_values(b_fmt)
    K = A.shape[1]
    total = Fraction(0)
    for k0 in range(0, K, 128):
        kb = k0 // 128
        part = sum(Fraction(va[A[m, k]]) * Fraction(vb[B[n, k]]) for k in range(k0, min(k0 + 128, K)))
        total += part * Fraction(2) ** (int(sa[kb, m]) - 127) * Fraction(2) ** (int(sb[n // 128, kb]) - 127)
    return total


@pytest.mark.parametrize("a_fmt,b_fmt,K", [(E4M3, E4M3, 272), (E5M2, E4M3, 144), (E4M3, E5M2, 128), (E5M2, E5M2, 16)])
def test_matches_exact_rational(a_fmt, b_fmt, K):
    rng = np.random.default_rng(K + 10 * a_fmt + 20 * b_fmt)
    M, N = 3, 131                      # N spans two 128-row scale blocks of B
    A = _codes(rng, a_fmt, (M, K))
    B = _codes(rng, b_fmt, (N, K))
    kb = (K + 127) // 128
    sa = _scales(rng, (kb, M))
    sb = _scales(rng, (2, kb))
    D, R, S = oracle.gemm_nt_blockscaled(A, B, sa, sb, a_fmt, b_fmt)
    for m in range(M):
        for n in (0, 1, 127, 128, 130):
            ex = _exact_element(A, B, sa, sb, m, n, a_fmt, b_fmt)
            assert D[m, n] == bf16_nearest_even(ex), (m, n)
            assert abs(Fraction(R[m, n]) - ex) <= abs(ex) * Fraction(1, 2 ** 50)


def test_scale_shift_invariance():
    """Doubling the A values of one (row, K block) while halving that block's
    scale, and likewise for one (128-row block, K block) of B, changes nothing;
    an index mix-up anywhere in the scale lookup breaks this."""
    rng = np.random.default_rng(3)
    M, N, K = 5, 260, 400
    kb = 4
    A = _codes(rng, E4M3, (M, K), hi_exp=12)
    B = _codes(rng, E4M3, (N, K), hi_exp=12)
    sa = _scales(rng, (kb, M), 123, 131)
    sb = _scales(rng, (3, kb), 123, 131)
    D0, R0, _ = oracle.gemm_nt_blockscaled(A, B, sa, sb)
    for (m, b) in [(0, 0), (2, 1), (4, 3)]:
        A2, sa2 = A.copy(), sa.copy()
        ks = slice(128 * b, min(128 * b + 128, K))
        A2[m, ks] = A2[m, ks] + (1 << 3)        # exponent + 1: value x 2
        sa2[b, m] -= 1
        D1, R1, _ = oracle.gemm_nt_blockscaled(A2, B, sa2, sb)
        assert np.array_equal(D0, D1) and np.array_equal(R0, R1), (m, b)
        # the same change without the scale correction must move row m only
        D2, _, _ = oracle.gemm_nt_blockscaled(A2, B, sa, sb)
        changed = np.unique(np.nonzero(D2 != D0)[0])
        assert list(changed) == [m]
    for (nb, b) in [(0, 2), (2, 0)]:
        B2, sb2 = B.copy(), sb.copy()
        rows = slice(128 * nb, min(128 * nb + 128, N))
        ks = slice(128 * b, min(128 * b + 128, K))
        B2[rows, ks] = B2[rows, ks] + (1 << 3)
        sb2[nb, b] -= 1
        D1, R1, _ = oracle.gemm_nt_blockscaled(A, B2, sa, sb2)
        assert np.array_equal(D0, D1) and np.array_equal(R0, R1), (nb, b)


@pytest.mark.parametrize("ea,eb", [(0, 0), (3, -2), (-5, 1)])
def test_uniform_scales_equal_per_tensor(ea, eb):
    rng = np.random.default_rng(5)
    M, N, K = 7, 140, 300
    A = rng.integers(0, 256, size=(M, K)).astype(np.uint8)
    B = rng.integers(0, 256, size=(N, K)).astype(np.uint8)
    A[(A & 0x7F) == 0x7F] = 0                  # no NaN codes
    B[(B & 0x7F) == 0x7F] = 0
    sa = np.full((3, M), 127 + ea, np.uint8)
    sb = np.full((2, 3), 127 + eb, np.uint8)
    D, R, S = oracle.gemm_nt_blockscaled(A, B, sa, sb)
    D1, R1, S1, _ = oracle.gemm_nt(A, B, sa=2.0 ** ea, sb=2.0 ** eb)
    assert np.array_equal(D, D1)
    np.testing.assert_allclose(R, R1, rtol=1e-15, atol=0)
    np.testing.assert_allclose(S, S1 * 2.0 ** (ea + eb), rtol=1e-15, atol=0)


def test_nan_scale_poisons_only_its_rows():
    rng = np.random.default_rng(6)
    M, N, K = 4, 200, 256
    A = _codes(rng, E4M3, (M, K))
    B = _codes(rng, E4M3, (N, K))
    sa = np.full((2, M), 127, np.uint8)
    sb = np.full((2, 2), 127, np.uint8)
    sa[1, 2] = 255                              # row 2, K block 1
    sb[1, 0] = 255                              # B rows 128..199, K block 0
    D, R, _ = oracle.gemm_nt_blockscaled(A, B, sa, sb)
    nan = np.isnan(R)
    assert nan[2, :].all() and nan[:, 128:].all()
    assert not nan[[0, 1, 3], :128].any()
    assert (D[nan] == 0x7FC0).all()


def test_points_equal_full():
    rng = np.random.default_rng(8)
    M, N, K = 9, 150, 208
    A = _codes(rng, E4M3, (M, K))
    B = _codes(rng, E4M3, (N, K))
    sa = _scales(rng, (2, M))
    sb = _scales(rng, (2, 2))
    D, R, S = oracle.gemm_nt_blockscaled(A, B, sa, sb)
    ii = rng.integers(0, M, 40)
    jj = rng.integers(0, N, 40)
    Dp, Rp, Sp = oracle.gemm_nt_blockscaled_points(A, B, sa, sb, ii, jj)
    assert np.array_equal(Dp, D[ii, jj]) and np.array_equal(Rp, R[ii, jj]) and np.array_equal(Sp, S[ii, jj])


def test_scale_leading_dimensions():
    """scale_a with extra columns (row stride > M) and scale_b with extra K blocks."""
    rng = np.random.default_rng(9)
    M, N, K = 3, 20, 130
    A = _codes(rng, E4M3, (M, K))
    B = _codes(rng, E4M3, (N, K))
    sa = _scales(rng, (2, M))
    sb = _scales(rng, (1, 2))
    sa_wide = np.full((2, 16), 200, np.uint8)
    sa_wide[:, :M] = sa
    sb_wide = np.full((1, 8), 200, np.uint8)
    sb_wide[:, :2] = sb
    D0, R0, _ = oracle.gemm_nt_blockscaled(A, B, sa, sb)
    D1, R1, _ = oracle.gemm_nt_blockscaled(A, B, sa_wide, sb_wide)
    assert np.array_equal(D0, D1) and np.array_equal(R0, R1)


def test_masked_grouped_equals_per_group_dense_and_leaves_rows():
    """The grouped block-scaled oracle is the per-group dense block-scaled
    oracle (pinned above) on rows < clamp(m_g), and leaves every other row."""
    rng = np.random.default_rng(17)
    G, cap, N, K = 4, 40, 150, 272
    A = _codes(rng, E4M3, (G, cap, K))
    B = _codes(rng, E4M3, (G, N, K))
    sa = _scales(rng, (G, 3, 44))
    sb = _scales(rng, (G, 2, 4))
    mm = np.array([0, 40, 17, 99], np.int32)
    init = np.full((G, cap, N), 0xBEEF, np.uint16)
    D, R, S = oracle.grouped_masked_blockscaled(A, B, mm, sa, sb, D_init=init)
    for g in range(G):
        m = min(max(int(mm[g]), 0), cap)
        if m:
            Dg, Rg, Sg = oracle.gemm_nt_blockscaled(A[g, :m], B[g], sa[g], sb[g])
            assert np.array_equal(D[g, :m], Dg) and np.array_equal(R[g, :m], Rg)
        assert (D[g, m:] == 0xBEEF).all()


def test_contig_grouped_equals_per_expert_dense_and_skips_padding():
    """Each valid row of the contiguous block-scaled oracle is the dense
    block-scaled oracle (pinned above) on that row with its expert's weights and
    scales; padding rows and out-of-range indices keep the initial value."""
    rng = np.random.default_rng(19)
    G, N, K = 3, 140, 272
    M = 9
    A = _codes(rng, E4M3, (M, K))
    B = _codes(rng, E4M3, (G, N, K))
    sa = _scales(rng, (3, 12))
    sb = _scales(rng, (G, 2, 4))
    gi = np.array([0, 0, -1, 2, 2, 1, 7, 1, -3], np.int32)
    init = np.full((M, N), 0xBEEF, np.uint16)
    D, R, S = oracle.grouped_contig_blockscaled(A, B, gi, sa, sb, D_init=init)
    for r in range(M):
        e = int(gi[r])
        if 0 <= e < G:
            Dr, Rr, _ = oracle.gemm_nt_blockscaled(A[r:r + 1], B[e], sa[:, r:r + 1], sb[e])
            assert np.array_equal(D[r], Dr[0]) and np.array_equal(R[r], Rr[0])
        else:
            assert (D[r] == 0xBEEF).all()
