"""Pins for the oracle's dense and grouped GEMMs (CPU only).

What the oracle computes: the naive per-element inner product ("DeepGEMM: FP8
matrix-multiply kernels on Hopper Tensor Cores", section 2.1) over decoded FP8
values (section 3.1) with the per-tensor scale applied at the output (sections
3.1, 5.2), rounded to BF16; grouped forms per "One transpose, half the compute:
the DeepSeek SwapAB story", sections 2 and 3.1-3.3.

Each pin is independent of the oracle's code: exact rational arithmetic on
torch-decoded values, numpy float64 matmul, closed forms, invariants.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests._exact import exact_gemm, fp8_values

E4M3, E5M2 = oracle.E4M3, oracle.E5M2


def _finite_codes(fmt):
    t = fp8_values(fmt)
    return np.array([c for c in range(256) if math.isfinite(t[c])], dtype=np.uint8)


def _torch_decode(codes, fmt):
    dt = torch.float8_e4m3fn if fmt == E4M3 else torch.float8_e5m2
    return torch.from_numpy(np.ascontiguousarray(codes)).view(dt).double().numpy()


# ---------------------------------------------------------------------------
# Brute force on tiny inputs
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("a_fmt,b_fmt", [(E4M3, E4M3), (E5M2, E5M2), (E4M3, E5M2), (E5M2, E4M3)])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_dense_matches_exact_rational(a_fmt, b_fmt, seed):
    rng = np.random.default_rng(100 + seed)
    M, N, K = 5, 6, 48
    # every finite code, including subnormals and the extremes
    A = rng.choice(_finite_codes(a_fmt), size=(M, K))
    B = rng.choice(_finite_codes(b_fmt), size=(N, K))
    D, R, S, EX = oracle.gemm_nt(A, B, a_fmt, b_fmt, want_exact=True)
    assert np.array_equal(D, exact_gemm(A, B, a_fmt, b_fmt))


@pytest.mark.parametrize("sa,sb", [(0.5, 4.0), (2.0 ** -7, 1.0), (1.0, 2.0 ** 9)])
def test_dense_power_of_two_scales_exact(sa, sb):
    rng = np.random.default_rng(11)
    A = rng.choice(_finite_codes(E4M3), size=(4, 32))
    B = rng.choice(_finite_codes(E4M3), size=(3, 32))
    D, _, _, _ = oracle.gemm_nt(A, B, sa=sa, sb=sb)
    assert np.array_equal(D, exact_gemm(A, B, E4M3, E4M3, sa, sb))


def test_dense_nonfinite_inputs_follow_ieee():
    A = np.full((3, 16), 0x38, dtype=np.uint8)       # 1.0
    B = np.full((4, 16), 0x38, dtype=np.uint8)
    A[0, 3] = 0x7F                                   # NaN in row 0
    B[1, 5] = 0x7F                                   # NaN in column 1
    D, R, S, _ = oracle.gemm_nt(A, B)
    assert np.array_equal(D, exact_gemm(A, B, E4M3, E4M3))
    assert D[0, 0] == 0x7FC0 and D[2, 1] == 0x7FC0 and D[2, 0] == oracle.bf16_rne(16.0)
    # E5M2 infinities: inf*1 -> inf, inf + -inf -> NaN, 0*inf -> NaN
    A2 = np.full((3, 8), 0x3C, dtype=np.uint8)
    B2 = np.full((2, 8), 0x3C, dtype=np.uint8)
    A2[0, 0] = 0x7C
    A2[1, 0], A2[1, 1] = 0x7C, 0xFC
    A2[2, 0] = 0x7C
    B2[1, 0] = 0x00
    D2, _, _, _ = oracle.gemm_nt(A2, B2, E5M2, E5M2)
    assert np.array_equal(D2, exact_gemm(A2, B2, E5M2, E5M2))
    assert D2[0, 0] == 0x7F80 and D2[1, 0] == 0x7FC0 and D2[2, 1] == 0x7FC0


# ---------------------------------------------------------------------------
# Library routine on decoded values (numpy float64 matmul)
# ---------------------------------------------------------------------------

def test_dense_r_matches_numpy_float64_matmul_e4m3():
    """For E4M3 every partial sum is exact in FP64 in any order, so the
    oracle's R must equal numpy's float64 matmul bit for bit (a transposed
    operand or a dropped term would show)."""
    w = workloads.dense_random(67, 45, 640, seed=3)
    D, R, S, EX = oracle.gemm_nt(w.A, w.B, want_exact=True)
    a = _torch_decode(w.A, E4M3)
    b = _torch_decode(w.B, E4M3)
    assert np.array_equal(R, a @ b.T)
    assert np.array_equal(S, np.abs(a) @ np.abs(b).T)
    assert (EX == 1).all()
    D2, R2, _, _ = oracle.gemm_nt(w.A, w.B, sa=1.25, sb=0.75)
    assert np.array_equal(R2, (a @ b.T) * (1.25 * 0.75))


def test_dense_e5m2_close_to_numpy():
    w = workloads.dense_random(33, 29, 512, seed=4, a_fmt=E5M2, b_fmt=E5M2)
    _, R, S, EX = oracle.gemm_nt(w.A, w.B, E5M2, E5M2, want_exact=True)
    ref = _torch_decode(w.A, E5M2) @ _torch_decode(w.B, E5M2).T
    assert np.all(np.abs(R - ref) <= 1e-12 * S)
    assert (EX == 1).all()    # N(0,1) data: no rounding at all in FP64


def _exact_dot(a_codes, b_codes, a_fmt, b_fmt):
    va, vb = fp8_values(a_fmt), fp8_values(b_fmt)
    return sum((Fraction(va[int(x)]) * Fraction(vb[int(y)]) for x, y in zip(a_codes, b_codes)), Fraction(0))


def test_exactness_flag_reports_rounded_fp64_sums():
    """E5M2 products reach from 2^-32 (the smallest subnormal squared) to
    57344^2 = 0xC4000000: their sum needs up to 64 significant bits, more than
    FP64's 53, so the oracle's FP64 sum then rounds and its exactness flag must
    say 0.  Built cases (57344 at k = 0 against a small term at k = 9):
      57344^2 + 2^-32  (2^-16 * 2^-16): 64 bits       -> rounded, flag 0
      57344^2 + 2^-30  (2^-16 * 2^-14): 62 bits       -> rounded, flag 0
      57344^2 + 2^-28  (2^-14 * 2^-14): 60 bits       -> rounded, flag 0
      57344^2 + 2^-16  (2^-16 * 1.0):   48 bits       -> exact,   flag 1
      57344^2 + 2^-14  (2^-14 * 1.0):   46 bits       -> exact,   flag 1
    The flag is checked against exact rational sums of torch-decoded values."""
    K = 16
    A = np.zeros((2, K), np.uint8)
    B = np.zeros((3, K), np.uint8)
    A[:, 0] = 0x7B                       # 57344
    B[:, 0] = 0x7B
    A[0, 9], A[1, 9] = 0x01, 0x04        # 2^-16, 2^-14
    B[0, 9], B[1, 9], B[2, 9] = 0x01, 0x3C, 0x04   # 2^-16, 1.0, 2^-14
    D, R, S, EX = oracle.gemm_nt(A, B, E5M2, E5M2, want_exact=True)
    assert EX.tolist() == [[0, 1, 0], [0, 1, 0]]
    for i in range(2):
        for j in range(3):
            exact = _exact_dot(A[i], B[j], E5M2, E5M2)
            assert (Fraction(float(R[i, j])) == exact) == bool(EX[i, j] == 1)
    # the rounded sums lose exactly the small term
    assert R[0, 0] == 57344.0 ** 2 and R[1, 2] == 57344.0 ** 2


@pytest.mark.parametrize("a_fmt,b_fmt", [(E5M2, E5M2), (E4M3, E5M2), (E5M2, E4M3)])
def test_exactness_flag_matches_exact_arithmetic(a_fmt, b_fmt):
    """Codes drawn from every finite value of the formats: the flag is 1
    exactly where the FP64 result equals the exact rational sum.  E5M2 x E5M2
    products span 64 bits, so both outcomes occur; E4M3 x E5M2 products span
    2^-25 .. 2^24.6, about 50 bits, so those sums are almost always exact."""
    rng = np.random.default_rng(7 + 3 * a_fmt + b_fmt)
    M, N, K = 7, 9, 24
    A = rng.choice(_finite_codes(a_fmt), size=(M, K))
    B = rng.choice(_finite_codes(b_fmt), size=(N, K))
    _, R, _, EX = oracle.gemm_nt(A, B, a_fmt, b_fmt, want_exact=True)
    got = np.zeros((M, N), bool)
    for i in range(M):
        for j in range(N):
            got[i, j] = Fraction(float(R[i, j])) == _exact_dot(A[i], B[j], a_fmt, b_fmt)
    assert np.array_equal(EX == 1, got)
    assert got.any()
    if a_fmt == b_fmt == E5M2:
        assert (~got).any()


# ---------------------------------------------------------------------------
# Closed forms
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("K", [128, 256, 1280, 4096, 7168, 14336])
@pytest.mark.parametrize("fmt,one", [(E4M3, 0x38), (E5M2, 0x3C)])
def test_all_ones_gives_K(K, fmt, one):
    A = np.full((3, K), one, dtype=np.uint8)
    B = np.full((2, K), one, dtype=np.uint8)
    D, R, _, _ = oracle.gemm_nt(A, B, fmt, fmt)
    assert (R == K).all()
    f = torch.tensor([float(K)], dtype=torch.float32).to(torch.bfloat16).view(torch.int16).item() & 0xFFFF
    assert (D == f).all()


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_identity_B_returns_A(fmt):
    K = 64
    codes = _finite_codes(fmt)
    rng = np.random.default_rng(5)
    A = rng.choice(codes, size=(20, K))
    one = 0x38 if fmt == E4M3 else 0x3C
    B = np.zeros((K, K), dtype=np.uint8)
    np.fill_diagonal(B, one)
    D, R, _, _ = oracle.gemm_nt(A, B, fmt, fmt)
    ref = _torch_decode(A, fmt)
    assert np.array_equal(R, ref)   # +0 and -0 compare equal
    refbits = torch.from_numpy(ref.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nz = ref != 0
    assert np.array_equal(D[nz], refbits[nz])


def test_max_magnitude():
    K = 4096
    A = np.full((2, K), 0x7E, dtype=np.uint8)     # 448
    B = np.full((2, K), 0x7E, dtype=np.uint8)
    B[1] = 0xFE                                   # -448
    D, R, _, _ = oracle.gemm_nt(A, B)
    assert R[0, 0] == 822083584.0 == 49 * 2.0 ** 24
    assert R[0, 1] == -822083584.0
    assert D[0, 0] == 0x4E44 and D[0, 1] == 0xCE44   # 49*2^24 = 1.53125 * 2^29


def test_one_hot_lands_on_its_element():
    M, N, K = 7, 9, 256
    A = np.zeros((M, K), dtype=np.uint8)
    B = np.zeros((N, K), dtype=np.uint8)
    A[3, 200] = 0x40        # 2.0 in E4M3
    B[5, 200] = 0x48        # 4.0 in E4M3
    D, R, _, _ = oracle.gemm_nt(A, B)
    expect = np.zeros((M, N))
    expect[3, 5] = 8.0
    assert np.array_equal(R, expect)


def test_rounding_ties_at_the_output():
    # row: 1*1 + (2^-8)*1 ; 1*1 + (3*2^-8)*1
    A = np.zeros((2, 32), dtype=np.uint8)
    A[:, 0] = 0x38
    A[0, 1] = 0x02          # 2 * 2^-9 = 2^-8
    A[1, 1] = 0x06          # 6 * 2^-9 = 3 * 2^-8
    B = np.zeros((1, 32), dtype=np.uint8)
    B[0, :2] = 0x38
    D, R, _, _ = oracle.gemm_nt(A, B)
    assert R[0, 0] == 1 + 2.0 ** -8 and D[0, 0] == 0x3F80
    assert R[1, 0] == 1 + 3 * 2.0 ** -8 and D[1, 0] == 0x3F82


# ---------------------------------------------------------------------------
# Invariants
# ---------------------------------------------------------------------------

def test_swap_identity_is_transpose():
    w = workloads.dense_random(19, 23, 160, seed=6)
    D1, R1, _, _ = oracle.gemm_nt(w.A, w.B)
    D2, R2, _, _ = oracle.gemm_nt(w.B, w.A)
    assert np.array_equal(D1, D2.T) and np.array_equal(R1, R2.T)


def test_row_permutation_permutes_output():
    w = workloads.dense_random(31, 17, 96, seed=9)
    perm = np.random.default_rng(1).permutation(31)
    D1, _, _, _ = oracle.gemm_nt(w.A, w.B)
    D2, _, _, _ = oracle.gemm_nt(w.A[perm], w.B)
    assert np.array_equal(D1[perm], D2)


def test_thread_count_does_not_change_results():
    w = workloads.dense_random(40, 33, 256, seed=10, a_fmt=E5M2, b_fmt=E4M3)
    D1, R1, _, _ = oracle.gemm_nt(w.A, w.B, E5M2, E4M3, threads=1)
    D2, R2, _, _ = oracle.gemm_nt(w.A, w.B, E5M2, E4M3, threads=7)
    assert np.array_equal(D1, D2) and np.array_equal(R1, R2)


def test_points_equal_full():
    w = workloads.dense_random(50, 40, 384, seed=12)
    D, R, S, _ = oracle.gemm_nt(w.A, w.B, sa=0.7, sb=1.3)
    rng = np.random.default_rng(2)
    ii = rng.integers(0, 50, 200)
    jj = rng.integers(0, 40, 200)
    Dp, Rp, Sp, _ = oracle.gemm_nt_points(w.A, w.B, ii, jj, sa=0.7, sb=1.3)
    assert np.array_equal(Dp, D[ii, jj]) and np.array_equal(Rp, R[ii, jj]) and np.array_equal(Sp, S[ii, jj])


def test_empty_shapes():
    A = np.zeros((0, 32), dtype=np.uint8)
    B = np.zeros((5, 32), dtype=np.uint8)
    D, _, _, _ = oracle.gemm_nt(A, B)
    assert D.shape == (0, 5)
    # K = 0: the empty sum is zero
    D, R, _, _ = oracle.gemm_nt(np.zeros((2, 0), np.uint8), np.zeros((3, 0), np.uint8))
    assert (R == 0).all() and (D == 0).all()


# ---------------------------------------------------------------------------
# Grouped forms
# ---------------------------------------------------------------------------

SENT = 0xDEAD


def test_masked_matches_exact_and_leaves_rows_untouched():
    G, cap, N, K = 4, 6, 5, 32
    w = workloads.masked_random(G, cap, N, K, seed=21, m_values=[0, 1, 6, 3])
    D, R, S, _ = oracle.grouped_masked(w.A, w.B, w.masked_m, w.sb, sa=0.5,
                                       D_init=np.full((G, cap, N), SENT, np.uint16))
    for g in range(G):
        m = int(w.masked_m[g])
        if m:
            ref = exact_gemm(w.A[g, :m], w.B[g], E4M3, E4M3, 0.5, w.sb[g])
            assert np.array_equal(D[g, :m], ref)
        assert (D[g, m:] == SENT).all()
        assert np.isnan(R[g, m:]).all()


def test_masked_clamps_counts():
    G, cap, N, K = 3, 4, 3, 16
    w = workloads.masked_random(G, cap, N, K, seed=22, m_values=[-5, 99, 2])
    D, _, _, _ = oracle.grouped_masked(w.A, w.B, w.masked_m, w.sb,
                                       D_init=np.full((G, cap, N), SENT, np.uint16))
    assert (D[0] == SENT).all()
    # m = 99 clamps to cap = 4, and rows >= the generator's own clamp are NaN rows
    assert not (D[1] == SENT).any()
    assert (D[2, 2:] == SENT).all() and not (D[2, :2] == SENT).any()


def test_masked_equals_per_group_dense():
    G, cap, N, K = 3, 40, 24, 256
    w = workloads.masked_random(G, cap, N, K, seed=23, m_values=[40, 17, 1])
    D, R, _, _ = oracle.grouped_masked(w.A, w.B, w.masked_m, w.sb, sa=1.5)
    for g in range(G):
        m = int(w.masked_m[g])
        Dg, Rg, _, _ = oracle.gemm_nt(w.A[g, :m], w.B[g], sa=1.5, sb=float(w.sb[g]))
        assert np.array_equal(D[g, :m], Dg) and np.array_equal(R[g, :m], Rg)


def test_contig_matches_exact_and_skips_padding():
    G, N, K = 3, 4, 32
    w = workloads.contig_random(tokens=5, topk=1, G=G, N=N, K=K, seed=31, align=4, counts=[2, 0, 3])
    assert w.A.shape[0] == 4 + 0 + 4
    D, R, _, _ = oracle.grouped_contig(w.A, w.B, w.grp_idx, w.sb, sa=2.0,
                                       D_init=np.full((w.A.shape[0], N), SENT, np.uint16))
    for r in range(w.A.shape[0]):
        g = int(w.grp_idx[r])
        if g < 0:
            assert (D[r] == SENT).all() and np.isnan(R[r]).all()
        else:
            ref = exact_gemm(w.A[r:r + 1], w.B[g], E4M3, E4M3, 2.0, w.sb[g])
            assert np.array_equal(D[r:r + 1], ref)


def test_contig_out_of_range_index_is_padding():
    G, N, K = 2, 3, 16
    A = np.full((3, K), 0x38, np.uint8)
    B = np.full((G, N, K), 0x38, np.uint8)
    gi = np.array([1, 2, -7], np.int32)
    D, _, _, _ = oracle.grouped_contig(A, B, gi, np.ones(G, np.float32),
                                       D_init=np.full((3, N), SENT, np.uint16))
    assert (D[0] == oracle.bf16_rne(16.0)).all()
    assert (D[1] == SENT).all() and (D[2] == SENT).all()


def test_e4m3_exactness_flag_at_full_K():
    """Config-sized K: the FP64 sum equals the exact integer sum for E4M3."""
    w = workloads.dense_random(4, 4, 14336, seed=40)
    _, _, _, EX = oracle.gemm_nt(w.A, w.B, want_exact=True)
    assert (EX == 1).all()
