"""GPU parity of the block-scaled dense FP8 GEMM (fp8_gemm_nt_blockscaled)
against the CPU oracle, through the C ABI.

Bit-exact pins: uniform block scales reproduce the per-tensor entry point,
and doubling one (row, K block) of A or one (128-row block, K block) of B while
halving its scale changes nothing, which pins the kernel's scale indexing
without any tolerance.  Elsewhere the element-wise bound of tests/_parity.py
(random inputs with the capped truncation allowance).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests._parity import check, gpu_bits, hw_allowance_blockscaled, random_cap

pytestmark = pytest.mark.gpu

E4M3, E5M2 = 0, 1


def _lib():
    import fp8_gemm_amd
    return fp8_gemm_amd


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def run_bs(w, out=None):
    M, N, K = w.shape
    print(f"[blockscaled] M={M} N={N} K={K} fmt=({w.a_fmt},{w.b_fmt}) lds=({w.sa.shape[1]},{w.sb.shape[1]})", flush=True)
    d = _lib().gemm_nt_blockscaled(_dev(w.A), _dev(w.B), _dev(w.sa), _dev(w.sb), out=out,
                                   a_dtype=w.a_fmt, b_dtype=w.b_fmt)
    torch.cuda.synchronize()
    return gpu_bits(d)


def check_full(w, d):
    """Random inputs: the capped truncation allowance."""
    ref, r, s = oracle.gemm_nt_blockscaled(w.A, w.B, w.sa, w.sb, w.a_fmt, w.b_fmt)
    check(d, r, s, 1.0, ref_bits=ref, what=w.name,
          allowance=hw_allowance_blockscaled(w.A, w.B, w.a_fmt, w.b_fmt, w.sa, w.sb, s),
          max_allowed=random_cap(d.size, w.A.shape[1]))


@pytest.mark.parametrize("M,N,K,fa,fb", [
    (300, 264, 400, E4M3, E4M3),     # ragged M, N and a short last K block
    (130, 136, 272, E5M2, E4M3),
    (129, 392, 144, E4M3, E5M2),
    (17, 520, 384, E4M3, E4M3),      # few rows
    (513, 256, 128, E5M2, E5M2),     # one K block
])
def test_blockscaled_matches_oracle(M, N, K, fa, fb):
    w = workloads.dense_blockscaled(M, N, K, seed=M + N + K, a_fmt=fa, b_fmt=fb)
    check_full(w, run_bs(w))


# Seeded random shapes (few tokens, 128-row and 256-row tiles; N a multiple of
# 8, K a multiple of 16, random formats), three per kernel the planner picks:
# the plan is the recorded one (variant, K splits) and every output matches the
# oracle.
@pytest.mark.parametrize("M,N,K,fa,fb,variant,splits", [
    (16, 9120, 576, E5M2, E4M3, 4, 1), (10, 1696, 992, E5M2, E4M3, 4, 2), (29, 6896, 2432, E5M2, E5M2, 4, 1),
    (2128, 552, 2096, E5M2, E5M2, 2, 1), (3755, 728, 2304, E5M2, E4M3, 2, 1), (1616, 1288, 464, E4M3, E4M3, 2, 1),
    (1660, 7416, 592, E5M2, E4M3, 1, 1), (2321, 10600, 32, E4M3, E4M3, 1, 1), (2208, 5016, 608, E4M3, E4M3, 1, 1),
])
def test_blockscaled_random_shapes(M, N, K, fa, fb, variant, splits):
    p = _lib().plan(3, M, N, K)
    assert (p.variant, p.k_splits) == (variant, splits)
    w = workloads.dense_blockscaled(M, N, K, seed=2 * M + N + K, a_fmt=fa, b_fmt=fb)
    check_full(w, run_bs(w))


@pytest.mark.parametrize("M,N,K,fa,fb", [
    (4000, 3000, 528, E4M3, E4M3),      # M, N and K tails (K = 4 * 128 + 16)
    (3968, 3840, 1040, E5M2, E4M3),
])
def test_blockscaled_256_tiles_full(M, N, K, fa, fb):
    """The 256 x 256 tiles (the plan picks them for these shapes; their ring
    stores each wave's token rows permuted so that a lane's row scales are
    consecutive bytes) with partial tiles on every edge: the whole output."""
    assert _lib().plan(3, M, N, K).variant == 1
    w = workloads.dense_blockscaled(M, N, K, seed=M + N + K, a_fmt=fa, b_fmt=fb)
    check_full(w, run_bs(w))


def test_padding_scales_are_never_used():
    """Scale arrays with padding columns holding the NaN code (255): rows of A
    past M and K blocks past the last read nothing that reaches the output."""
    w = workloads.dense_blockscaled(257, 200, 400, seed=21, lds_pad=9, pad_code=255)
    d = run_bs(w)
    check_full(w, d)
    assert not ((d & 0x7F80) == 0x7F80).any(), "a padding scale reached the output"


def test_uniform_scales_equal_per_tensor_entry_point():
    """All scales 2^ea (A) and 2^eb (B): bit-identical to fp8_gemm_nt with
    scale_a = 2^ea, scale_b = 2^eb."""
    f = _lib()
    w = workloads.dense_random(300, 520, 400, seed=22)
    for ea, eb in [(0, 0), (3, -5)]:
        kb = 4
        sa = np.full((kb, 300), 127 + ea, np.uint8)
        sb = np.full((5, 4), 127 + eb, np.uint8)
        wb = workloads.BlockScaled(w.A, w.B, sa, sb, name=f"uniform {ea},{eb}")
        d1 = run_bs(wb)
        d0 = f.gemm_nt(_dev(w.A), _dev(w.B), torch.tensor([2.0 ** ea], device="cuda"),
                       torch.tensor([2.0 ** eb], device="cuda"), a_dtype=E4M3, b_dtype=E4M3)
        torch.cuda.synchronize()
        assert np.array_equal(d1, gpu_bits(d0)), (ea, eb)


@pytest.mark.parametrize("M,N,a_rows,b_blocks", [
    (260, 300, [(0, 0), (131, 2), (259, 3)], [(0, 1), (2, 3)]),
    (3968, 3840, [(0, 0), (7, 1), (136, 2), (2063, 3), (3967, 0)], [(0, 1), (29, 3)]),   # 256-row tiles
])
def test_scale_shift_is_bit_exact(M, N, a_rows, b_blocks):
    """Doubling the values of one (row, K block) of A and decrementing its
    scale, or the same for one (128-row block, K block) of B, leaves the GPU
    output bit-identical; the uncorrected change moves only the affected rows."""
    rng = np.random.default_rng(23)
    K = 400
    e = rng.integers(1, 13, size=(M, K))
    A = ((rng.integers(0, 2, size=(M, K)) << 7) | (e << 3) | rng.integers(0, 8, size=(M, K))).astype(np.uint8)
    e = rng.integers(1, 13, size=(N, K))
    B = ((rng.integers(0, 2, size=(N, K)) << 7) | (e << 3) | rng.integers(0, 8, size=(N, K))).astype(np.uint8)
    sa = rng.integers(112, 118, size=(4, M)).astype(np.uint8)
    sb = rng.integers(112, 118, size=((N + 127) // 128, 4)).astype(np.uint8)
    base = run_bs(workloads.BlockScaled(A, B, sa, sb, name="base"))
    for (m, b) in a_rows:
        A2, sa2 = A.copy(), sa.copy()
        ks = slice(128 * b, min(128 * b + 128, K))
        A2[m, ks] += 8
        sa2[b, m] -= 1
        assert np.array_equal(run_bs(workloads.BlockScaled(A2, B, sa2, sb, name="shift A")), base), (m, b)
        moved = run_bs(workloads.BlockScaled(A2, B, sa, sb, name="unshifted A"))
        assert list(np.unique(np.nonzero(moved != base)[0])) == [m]
    for (nb, b) in b_blocks:
        B2, sb2 = B.copy(), sb.copy()
        rows = slice(128 * nb, min(128 * nb + 128, N))
        ks = slice(128 * b, min(128 * b + 128, K))
        B2[rows, ks] += 8
        sb2[nb, b] -= 1
        assert np.array_equal(run_bs(workloads.BlockScaled(A, B2, sa, sb2, name="shift B")), base), (nb, b)


def test_nan_scale_poisons_only_its_outputs():
    w = workloads.dense_blockscaled(200, 300, 256, seed=24)
    w.sa[1, 5] = 255
    w.sb[2, 0] = 255                      # B rows 256..299
    d = run_bs(w)
    nan = ((d & 0x7F80) == 0x7F80) & ((d & 0x7F) != 0)
    assert nan[5, :].all() and nan[:, 256:].all()
    keep = np.ones_like(nan)
    keep[5, :] = False
    keep[:, 256:] = False
    assert not nan[keep].any()


def test_zero_sizes_and_empty_k():
    f = _lib()
    a = torch.zeros((0, 128), dtype=torch.uint8, device="cuda")
    b = torch.zeros((16, 128), dtype=torch.uint8, device="cuda")
    sa = torch.zeros((1, 4), dtype=torch.uint8, device="cuda")
    sb = torch.zeros((1, 4), dtype=torch.uint8, device="cuda")
    out = f.gemm_nt_blockscaled(a, b, sa, sb, a_dtype=E4M3, b_dtype=E4M3)
    assert out.shape == (0, 16)
    a = torch.zeros((40, 0), dtype=torch.uint8, device="cuda")
    b = torch.zeros((24, 0), dtype=torch.uint8, device="cuda")
    sa = torch.zeros((0, 40), dtype=torch.uint8, device="cuda")
    sb = torch.zeros((1, 0), dtype=torch.uint8, device="cuda")
    out = torch.full((40, 24), 3.0, dtype=torch.bfloat16, device="cuda")
    f.gemm_nt_blockscaled(a, b, sa, sb, out=out, a_dtype=E4M3, b_dtype=E4M3)
    torch.cuda.synchronize()
    assert (out == 0).all()


def test_blockscaled_4096_sampled():
    """The benchmarked block-scaled 4096^3 E4M3 case, sampled points, stated bound."""
    w = workloads.dense_blockscaled_square()
    d = run_bs(w)
    rng = np.random.default_rng(7)
    ii = np.concatenate([rng.integers(0, 4096, 2048), [0, 4095, 255, 256]])
    jj = np.concatenate([rng.integers(0, 4096, 2048), [4095, 0, 256, 255]])
    ref, r, s = oracle.gemm_nt_blockscaled_points(w.A, w.B, w.sa, w.sb, ii, jj)
    check(d[ii, jj], r, s, 1.0, ref_bits=ref, what=w.name)
