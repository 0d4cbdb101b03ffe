"""GPU parity of the BF16 comparison GEMM (bf16_gemm_nt) against the CPU oracle.

"DeepGEMM: FP8 matrix-multiply kernels on Hopper Tensor Cores", section 1.3: a
BF16 path kept beside the FP8 one for precision experiments.  Calls go through
the C ABI (via the Python binding).  Bit-exact where the exact result is a BF16
value (one-hot layout, identity weights, specials); elsewhere the element-wise
bound of tests/_parity.py, random inputs with the capped allowance for the
instruction's summation measured by the probe below.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests._parity import assert_within_bound, check, gpu_bits, hw_allowance_bf16, random_cap

pytestmark = pytest.mark.gpu


def _lib():
    import fp8_gemm_amd
    return fp8_gemm_amd


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda().view(torch.bfloat16)


def bf(v):
    return workloads.to_bf16(np.asarray(v, np.float32))


def run_bf16(A, B, out=None):
    print(f"[bf16] M={A.shape[0]} N={B.shape[0]} K={A.shape[1]}", flush=True)
    d = _lib().gemm_nt_bf16(_dev(A), _dev(B), out=out)
    torch.cuda.synchronize()
    return gpu_bits(d)


def _check_bf16(A, B, what):
    got = run_bf16(A, B)
    ref, r, s = oracle.gemm_nt_bf16(A, B)
    return check(got, r, s, 1.0, ref_bits=ref, what=what, allowance=hw_allowance_bf16(A, B, s),
                 max_allowed=random_cap(got.size, A.shape[1]))


@pytest.mark.parametrize("M,N,K", [(256, 256, 256), (300, 260, 392), (40, 96, 136)])
def test_one_hot_layout(M, N, K):
    """One product per output row at a distinct K position, every value a small
    integer: pins row, column and K placement, including the split of each
    fragment over two instructions."""
    rng = np.random.default_rng(M + N + K)
    n = min(M, N, K)
    rows, cols, ks = rng.permutation(M)[:n], rng.permutation(N)[:n], rng.permutation(K)[:n]
    A = np.zeros((M, K), np.uint16)
    B = np.zeros((N, K), np.uint16)
    va = rng.integers(1, 9, n)
    vb = rng.integers(1, 9, n)
    A[rows, ks] = bf(va)
    B[cols, ks] = bf(vb)
    ref, _, _ = oracle.gemm_nt_bf16(A, B)
    got = run_bf16(A, B)
    assert np.array_equal(got, ref), f"{int((got != ref).sum())} mismatches"


@pytest.mark.parametrize("M,K", [(64, 264), (300, 512)])
def test_identity_B_returns_A(M, K):
    """B = I (N = K): D = A bit for bit, so every K position of every row lands
    on its own output column."""
    rng = np.random.default_rng(K)
    A = bf(rng.standard_normal((M, K)).astype(np.float32))
    B = np.zeros((K, K), np.uint16)
    B[np.arange(K), np.arange(K)] = bf(1.0)
    got = run_bf16(A, B)
    assert np.array_equal(got, A)


# (distance d of the small product s from the large P = 2^16, s)
PROBE = [(1, 1.0 + 2.0 ** -7), (7, 1.0 + 2.0 ** -7), (8, 1.0 + 2.0 ** -7), (15, 1.0 + 2.0 ** -7),
         (16, 1.0 + 2.0 ** -7), (17, 1.0 + 2.0 ** -7), (24, 1.0 + 2.0 ** -7), (31, 1.0 + 2.0 ** -7),
         (1, 2.0 ** -6), (16, 2.0 ** -6), (8, 2.0 ** -6), (1, 3.0), (1, 0.5 + 2.0 ** -8),
         (32, 1.0 + 2.0 ** -7), (40, 2.0 ** -6), (63, 1.0 + 2.0 ** -7),
         (1, 0.5 + 3 * 2.0 ** -8), (1, -(0.5 + 3 * 2.0 ** -8)), (17, 0.5 + 3 * 2.0 ** -8),
         (9, 0.5 + 2.0 ** -8), (1, 2.0 ** -9), (1, 3 * 2.0 ** -9), (1, -(2.0 ** -9)), (1, -3 * 2.0 ** -9),
         (40, 3 * 2.0 ** -9), (40, 0.5 + 3 * 2.0 ** -8)]


def _model(P, s, same_instruction):
    """Predicted result of P + s - P: inside one instruction s is first cut
    toward zero to a multiple of 2^(E - 24), E = 16 the exponent of P; the sum
    is then rounded to FP32, nearest even, and P cancels exactly."""
    if same_instruction:
        q = 2.0 ** (16 - 24)
        s = np.trunc(s / q) * q
    return float(np.float32(np.float64(P) + np.float64(s))) - P


def test_bf16_instruction_numerics_probe():
    """Row r puts P = 256 * 256 at k = 0, a small product s at k = d and -P at
    k = 64 (the next 128-byte K step), so the exact result is s.  d >= 32 lies
    in the other instruction of the same K step (s meets P only in the FP32
    accumulator); d < 32 shares an instruction with P.

    Measured: within one instruction the products are aligned to the largest
    one, exponent E, and bits below 2^(E - 24) are cut toward zero (one bit
    beyond FP32's 24-bit significand is kept); the aligned sum is then rounded
    to FP32, nearest even.  So 1 + 2^-7 survives next to 2^16, 0.5 + 2^-8 and
    0.5 + 3 * 2^-8 are FP32 ties that round to even (0.5 and 0.515625), and
    3 * 2^-9 is cut to 2^-8, a tie that rounds to 0."""
    M, N, K = 64, 16, 128
    A = np.zeros((M, K), np.uint16)
    B = np.zeros((N, K), np.uint16)
    B[:, :] = bf(1.0)
    B[:, 0] = bf(256.0)
    B[:, 64] = bf(256.0)
    for r, (d, s) in enumerate(PROBE):
        A[r, 0] = bf(256.0)
        A[r, d] = bf(s)
        A[r, 64] = bf(-256.0)
    got = torch.from_numpy(run_bf16(A, B).view(np.int16)).view(torch.bfloat16).double().numpy()
    for r, (d, s) in enumerate(PROBE):
        print(f"  d={d:2d} s={s!r}: got {got[r, 0]!r}, model {_model(65536.0, s, d < 32)!r}", flush=True)
    for r, (d, s) in enumerate(PROBE):
        assert (got[r] == got[r, 0]).all()
        assert got[r, 0] == _model(65536.0, s, d < 32), (d, s, got[r, 0])
    assert (got[len(PROBE):] == 0).all()


SHAPES = [(1, 1, 8), (1, 200, 128), (7, 64, 72), (16, 257, 120), (33, 255, 256), (64, 65, 8),
          (65, 64, 136), (127, 128, 200), (129, 257, 392), (255, 300, 640), (257, 255, 1032),
          (300, 520, 264), (513, 260, 128)]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_ragged_shapes(M, N, K):
    w = workloads.dense_bf16_random(M, N, K, seed=M * 7 + N * 3 + K)
    _check_bf16(w.A, w.B, f"bf16 {M}x{N}x{K}")


def test_bf16_4096_config_sampled():
    """The seeded 4096^3 BF16 configuration (the draws of the FP8 4096^3 case):
    the stated bound on every sampled element and on full rows through the
    tile boundaries."""
    w = workloads.dense_bf16_square()
    M, N, K = w.shape
    d = run_bf16(w.A, w.B)
    rng = np.random.default_rng(4096)
    ii = np.concatenate([rng.integers(0, M, 4000), np.zeros(N // 16, np.int64), np.full(N // 16, M - 1)])
    jj = np.concatenate([rng.integers(0, N, 4000), np.arange(0, N, 16), np.arange(7, N, 16)])
    ref, r, s = oracle.gemm_nt_bf16_points(w.A, w.B, ii, jj)
    assert_within_bound(d[ii, jj], r, s, 1.0, ref_bits=ref, what="bf16 4096^3 sampled")
    rows = np.array([0, 255, 256, 4095])
    Dr, Rr, Sr = oracle.gemm_nt_bf16(w.A[rows], w.B)
    assert_within_bound(d[rows], Rr, Sr, 1.0, ref_bits=Dr, what="bf16 4096^3 full rows")


def test_specials_propagate():
    M, N, K = 130, 260, 264
    w = workloads.dense_bf16_random(M, N, K, seed=5)
    A, B = w.A.copy(), w.B.copy()
    A[3, 17] = 0x7FC0                 # NaN: row 3 all NaN
    A[100, 200] = 0x7F80              # +inf in row 100 ...
    B[9, 200] = 0x0000                # ... times 0 in column 9: NaN there, +-inf elsewhere
    B[250, 5] = 0xFF80                # -inf: column 250
    got = run_bf16(A, B)
    ref, r, s = oracle.gemm_nt_bf16(A, B)
    check(got, r, s, 1.0, ref_bits=ref, what="bf16 specials", allowance=hw_allowance_bf16(A, B, s),
          max_allowed=random_cap(got.size, K))
    nan = lambda x: ((x & 0x7F80) == 0x7F80) & ((x & 0x7F) != 0)
    assert nan(got[3]).all() and nan(got[100, 9])


def test_strided_operands_and_output():
    M, N, K = 200, 136, 256
    w = workloads.dense_bf16_random(M, N, K, seed=12)
    A = np.zeros((M, K + 24), np.uint16)
    A[:, :K] = w.A
    B = np.zeros((N, K + 8), np.uint16)
    B[:, :K] = w.B
    big = torch.full((M, N + 40), -7.0, dtype=torch.bfloat16, device="cuda")
    out = big[:, :N]
    _lib().gemm_nt_bf16(_dev(A)[:, :K], _dev(B)[:, :K], out=out)
    torch.cuda.synchronize()
    ref, r, s = oracle.gemm_nt_bf16(w.A, w.B)
    check(gpu_bits(out), r, s, 1.0, ref_bits=ref, what="bf16 strided", allowance=hw_allowance_bf16(w.A, w.B, s),
          max_allowed=random_cap(out.numel(), K))
    assert (big[:, N:] == -7.0).all()


def test_zero_sizes_and_empty_k():
    f = _lib()
    e = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    b = torch.ones((32, 64), dtype=torch.bfloat16, device="cuda")
    assert f.gemm_nt_bf16(e, b).shape == (0, 32)
    a0 = torch.empty((40, 0), dtype=torch.bfloat16, device="cuda")
    b0 = torch.empty((24, 0), dtype=torch.bfloat16, device="cuda")
    out = torch.full((40, 24), 3.0, dtype=torch.bfloat16, device="cuda")
    f.gemm_nt_bf16(a0, b0, out=out)
    torch.cuda.synchronize()
    assert (out == 0).all()


def test_deterministic_repeats():
    w = workloads.dense_bf16_random(512, 384, 1024, seed=3)
    outs = [run_bf16(w.A, w.B) for _ in range(3)]
    assert all(np.array_equal(outs[0], o) for o in outs[1:])


def test_validation_through_binding():
    f = _lib()
    a = torch.ones((64, 12), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(f.Fp8GemmError) as e:
        f.gemm_nt_bf16(a, a)                        # K % 8
    assert e.value.status == -2
    with pytest.raises(TypeError):
        f.gemm_nt_bf16(torch.ones((8, 8), device="cuda"), torch.ones((8, 8), device="cuda"))
