"""GPU parity at the largest K the library accepts (the row-stride limit).

The kernels address each tile with 32-bit offsets from a 64-bit base; the
limit of 2^23 - 16 bytes per row keeps 256 rows of offsets below 2^31, so at
K = 2^23 - 16 a 256-row tile's last element sits 4112 bytes below 2^31.  The
operands are zero except for a few entries at both ends of K, in the first and
last rows; since zero columns add exactly nothing, the oracle runs on the
non-zero columns only and its sums are those of the full problem.
"""
import gc

import numpy as np
import pytest
import torch

import oracle
from tests._parity import assert_within_bound, gpu_bits

pytestmark = pytest.mark.gpu

KMAX = (1 << 23) - 16                      # bytes per row: FP8 elements
KMAX_BF16 = KMAX // 2


def _lib():
    import fp8_gemm_amd
    return fp8_gemm_amd


T4 = None


def code(v):
    global T4
    if T4 is None:
        T4 = oracle.decode_table(0)
    return int(np.flatnonzero(T4 == v)[0])


def _sparse(rows, K, seed, ks, dtype=np.uint8, values=None):
    """rows x K zeros with entries at columns ks in rows 0, 1, rows-2, rows-1
    and a few random rows."""
    rng = np.random.default_rng(seed)
    X = np.zeros((rows, K), dtype)
    rr = sorted(set([0, 1, rows - 2, rows - 1] + list(rng.integers(0, rows, 4))))
    for r in rr:
        for k in ks:
            X[r, k] = values[rng.integers(0, len(values))]
    return X


def _cols(K):
    return sorted(set([0, 16, 4096, K // 2, K - 1024, K - 48, K - 17, K - 16, K - 1]))


def _check_fp8(got, A, B, cols, what):
    Ac, Bc = np.ascontiguousarray(A[:, cols]), np.ascontiguousarray(B[:, cols])
    ref, r, s, _ = oracle.gemm_nt(Ac, Bc)
    assert np.abs(r).max() > 0
    assert_within_bound(got, r, s, 1.0, ref_bits=ref, what=what)


def _free():
    gc.collect()
    torch.cuda.empty_cache()


FP8_VALUES = [code(v) for v in (1.0, -2.0, 3.0, 0.5, -6.0, 1.5)]


@pytest.mark.parametrize("M", [130, 40])          # 128x256 tiles; decode kernel
def test_max_k_dense(M):
    K, N = KMAX, 24
    cols = _cols(K)
    A = _sparse(M, K, 1, cols, values=FP8_VALUES)
    B = _sparse(N, K, 2, cols, values=FP8_VALUES)
    f = _lib()
    print(f"[limits] dense M={M} N={N} K={K} variant {f.plan(0, M, N, K).variant}", flush=True)
    one = torch.ones(1, device="cuda")
    a, b = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()
    d = f.gemm_nt(a, b, one, one, a_dtype=0, b_dtype=0)
    torch.cuda.synchronize()
    got = gpu_bits(d)
    del a, b, d
    _free()
    _check_fp8(got, A, B, cols, f"dense M={M} at K={K}")


def test_max_k_contig_256_row_tile():
    """The contiguous form always tiles 256 rows: the descriptor of A covers
    256 * (2^23 - 16) = 2^31 - 4096 bytes."""
    K, N, M = KMAX, 16, 256
    cols = _cols(K)
    A = _sparse(M, K, 3, cols, values=FP8_VALUES)
    B = _sparse(N, K, 4, cols, values=FP8_VALUES)
    gi = np.zeros(M, np.int32)
    f = _lib()
    print(f"[limits] contig M={M} N={N} K={K}", flush=True)
    one = torch.ones(1, device="cuda")
    a, b = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda().reshape(1, N, K)
    out = torch.zeros((M, N), dtype=torch.bfloat16, device="cuda")
    f.grouped_gemm_contig(a, b, one, one, torch.from_numpy(gi).cuda(), out=out, a_dtype=0, b_dtype=0)
    torch.cuda.synchronize()
    got = gpu_bits(out)
    del a, b, out
    _free()
    _check_fp8(got, A, B, cols, f"contig at K={K}")


def test_max_k_masked():
    K, N, cap, m = KMAX, 16, 64, 40
    cols = _cols(K)
    A = _sparse(cap, K, 5, cols, values=FP8_VALUES)
    A[m:] = 0x7F                                   # rows past the count: NaN, never read
    B = _sparse(N, K, 6, cols, values=FP8_VALUES)
    f = _lib()
    print(f"[limits] masked cap={cap} m={m} N={N} K={K}", flush=True)
    one = torch.ones(1, device="cuda")
    a = torch.from_numpy(A).cuda().reshape(1, cap, K)
    b = torch.from_numpy(B).cuda().reshape(1, N, K)
    out = torch.zeros((1, cap, N), dtype=torch.bfloat16, device="cuda")
    mm = torch.tensor([m], dtype=torch.int32, device="cuda")
    f.grouped_gemm_masked(a, b, one, one, mm, out=out, expected_m=m, a_dtype=0, b_dtype=0)
    torch.cuda.synchronize()
    got = gpu_bits(out)[0]
    del a, b, out
    _free()
    assert (got[m:] == 0).all()
    _check_fp8(got[:m], A[:m], B, cols, f"masked at K={K}")


def test_max_k_bf16():
    K, M, N = KMAX_BF16, 130, 24
    cols = _cols(K)
    vals = [0x3F80, 0xC000, 0x4040, 0x3F00, 0xC0C0]   # 1, -2, 3, 0.5, -6
    A = _sparse(M, K, 7, cols, dtype=np.uint16, values=vals)
    B = _sparse(N, K, 8, cols, dtype=np.uint16, values=vals)
    f = _lib()
    print(f"[limits] bf16 M={M} N={N} K={K}", flush=True)
    a = torch.from_numpy(A.view(np.int16)).cuda().view(torch.bfloat16)
    b = torch.from_numpy(B.view(np.int16)).cuda().view(torch.bfloat16)
    d = f.gemm_nt_bf16(a, b)
    torch.cuda.synchronize()
    got = gpu_bits(d)
    del a, b, d
    _free()
    Ac, Bc = np.ascontiguousarray(A[:, cols]), np.ascontiguousarray(B[:, cols])
    ref, r, s = oracle.gemm_nt_bf16(Ac, Bc)
    assert_within_bound(got, r, s, 1.0, ref_bits=ref, what=f"bf16 at K={K}")


def test_k_past_the_limit_is_rejected():
    f = _lib()
    a = torch.zeros((8, KMAX + 16), dtype=torch.uint8, device="cuda")
    one = torch.ones(1, device="cuda")
    with pytest.raises(f.Fp8GemmError) as e:
        f.gemm_nt(a, a, one, one, a_dtype=0, b_dtype=0)
    assert e.value.status == -2
