"""Pins of the oracle's BF16 comparison path (DeepGEMM on Hopper, section 1.3:
a BF16 backend kept for precision experiments) against things other than
itself: torch's bfloat16 decode, numpy float64 matmul on decoded values, the
independently pinned FP8 oracle (every E4M3 / E5M2 value is a BF16 value),
closed forms, and IEEE special cases."""
import numpy as np
import pytest
import torch

import oracle
import workloads


def torch_bf16_values(bits):
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).double().numpy()


def bits_of(v):
    return int(workloads.to_bf16(np.array([v], np.float32))[0])


def test_decode_every_pattern_matches_torch():
    pats = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = torch_bf16_values(pats)
    got = np.array([oracle.bf16_value(int(p)) for p in pats])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.signbit(got[fin]), np.signbit(ref[fin]))   # -0 stays -0


def _nearest_bf16(d_bits, r):
    """True where BF16 d is a nearest BF16 value to r (one of its neighbours is
    never strictly closer)."""
    d = torch_bf16_values(d_bits)
    up = torch_bf16_values((d_bits.astype(np.int32) + 1).astype(np.uint16))
    dn = torch_bf16_values((d_bits.astype(np.int32) - 1).astype(np.uint16))
    err = np.abs(d - r)
    with np.errstate(invalid="ignore"):
        ok_up = ~(np.abs(up - r) < err)
        ok_dn = ~(np.abs(dn - r) < err)
    return ok_up & ok_dn


def test_random_matches_float64_matmul_transposed_operand():
    d = workloads.dense_bf16_random(37, 29, 264, seed=11)
    D, R, S = oracle.gemm_nt_bf16(d.A, d.B)
    a, b = torch_bf16_values(d.A), torch_bf16_values(d.B)
    ref = a @ b.T
    assert np.all(np.abs(R - ref) <= 1e-12 * S)
    assert np.allclose(S, np.abs(a) @ np.abs(b).T, rtol=1e-12)
    assert _nearest_bf16(D, R).all()
    # the result is not symmetric in the operands: A . B^T, not B . A^T
    D2, R2, _ = oracle.gemm_nt_bf16(d.B, d.A)
    assert np.array_equal(R2, R.T) and np.array_equal(D2, D.T)


@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_fp8_values_reduce_to_the_fp8_oracle(fmt):
    dt = torch.float8_e4m3fn if fmt == oracle.E4M3 else torch.float8_e5m2
    f8 = workloads.dense_random(24, 40, 200, seed=12, a_fmt=fmt, b_fmt=fmt)
    as_bf16 = lambda c: torch.from_numpy(c).view(dt).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    D, R, S = oracle.gemm_nt_bf16(as_bf16(f8.A), as_bf16(f8.B))
    D8, R8, S8, _ = oracle.gemm_nt(f8.A, f8.B, fmt, fmt, 1.0, 1.0)
    assert np.array_equal(D, D8) and np.array_equal(R, R8) and np.array_equal(S, S8)


def test_closed_forms():
    one = bits_of(1.0)
    # sum of K ones, rounded once: 257 lies halfway between 256 and 258 and
    # goes to the even mantissa (256); 259 lies halfway between 258 and 260
    # and goes to 260
    for K, want in ((256, 256.0), (257, 256.0), (259, 260.0), (1000, 1000.0)):
        A = np.full((1, K), one, np.uint16)
        D, R, _ = oracle.gemm_nt_bf16(A, A)
        assert R[0, 0] == K and torch_bf16_values(D)[0, 0] == want, K
    # every term counts and A's row index meets B's row index: D[i, j] =
    # sum_k (i + 1) * (k + 1) * (j + 1)
    M, N, K = 3, 4, 5
    A = np.array([[bits_of((i + 1) * (k + 1)) for k in range(K)] for i in range(M)], np.uint16)
    B = np.array([[bits_of(j + 1)] * K for j in range(N)], np.uint16)
    _, R, _ = oracle.gemm_nt_bf16(A, B)
    want = np.array([[(i + 1) * (j + 1) * K * (K + 1) / 2 for j in range(N)] for i in range(M)])
    assert np.array_equal(R, want)


def test_one_rounding_not_two():
    # 1 + 2^-8 + 2^-30 lies just above the BF16 tie 1 + 2^-8, so it rounds up to
    # 1 + 2^-7; an intermediate FP32 rounding would land on the tie and give 1.
    A = np.array([[bits_of(1.0), bits_of(2.0 ** -8), bits_of(2.0 ** -30)]], np.uint16)
    B = np.full((1, 3), bits_of(1.0), np.uint16)
    D, R, _ = oracle.gemm_nt_bf16(A, B)
    assert R[0, 0] == 1.0 + 2.0 ** -8 + 2.0 ** -30
    assert torch_bf16_values(D)[0, 0] == 1.0 + 2.0 ** -7


def test_special_values():
    inf, ninf, nan = 0x7F80, 0xFF80, 0x7FC0
    one, zero, two = bits_of(1.0), 0x0000, bits_of(2.0)
    big = 0x7F00                                  # 2^127
    rows = {
        "inf*0": ([inf, one], [zero, one], np.nan),
        "inf-inf": ([inf, ninf], [one, one], np.nan),
        "inf*2": ([inf, one], [two, one], np.inf),
        "nan": ([nan, one], [one, one], np.nan),
        "overflow": ([big, zero], [big, zero], np.inf),   # 2^254: finite in FP64, inf in BF16
        "subnormal": ([0x0001, zero], [bits_of(1024.0), zero], 2.0 ** -123),
    }
    for name, (a, b, want) in rows.items():
        D, R, _ = oracle.gemm_nt_bf16(np.array([a], np.uint16), np.array([b], np.uint16))
        got = torch_bf16_values(D)[0, 0]
        if np.isnan(want):
            assert np.isnan(got) and D[0, 0] == 0x7FC0, name
        else:
            assert got == want, name
    _, R, _ = oracle.gemm_nt_bf16(np.array([[big, zero]], np.uint16), np.array([[big, zero]], np.uint16))
    assert R[0, 0] == 2.0 ** 254


def test_points_equal_full():
    d = workloads.dense_bf16_random(50, 70, 136, seed=13)
    D, R, S = oracle.gemm_nt_bf16(d.A, d.B)
    rng = np.random.default_rng(0)
    ii = rng.integers(0, 50, 300)
    jj = rng.integers(0, 70, 300)
    Dp, Rp, Sp = oracle.gemm_nt_bf16_points(d.A, d.B, ii, jj)
    assert np.array_equal(Dp, D[ii, jj]) and np.array_equal(Rp, R[ii, jj]) and np.array_equal(Sp, S[ii, jj])


def test_empty_sizes():
    D, R, S = oracle.gemm_nt_bf16(np.zeros((0, 16), np.uint16), np.zeros((5, 16), np.uint16))
    assert D.shape == (0, 5)
    D, R, _ = oracle.gemm_nt_bf16(np.zeros((3, 0), np.uint16), np.zeros((4, 0), np.uint16))
    assert (R == 0).all() and (D == 0).all()


def test_workload_rounding():
    assert bits_of(1.0) == 0x3F80
    assert bits_of(1.0 + 2.0 ** -8) == 0x3F80            # tie -> even
    assert bits_of(1.0 + 3 * 2.0 ** -8) == 0x3F82        # tie -> even (up)
    d1 = workloads.dense_bf16_random(8, 8, 32, seed=3)
    d2 = workloads.dense_bf16_random(8, 8, 32, seed=3)
    assert np.array_equal(d1.A, d2.A) and np.array_equal(d1.B, d2.B)
