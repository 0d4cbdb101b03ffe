"""GPU parity of the dense few-token (M <= 64) path, the swap-AB decode kernel
with K split over 4 waves and per-wave LDS rings, against the CPU oracle,
through the C ABI.

Edges specific to it: fewer K blocks than waves (some waves have no work),
a short last K block, N not a multiple of the 16 weight rows per workgroup,
every token-block count (M = 1..64) with rings that wrap several times, mixed
formats, and the block-scaled form.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests._parity import check, gpu_bits

pytestmark = pytest.mark.gpu

E4M3, E5M2 = 0, 1


def _f():
    import fp8_gemm_amd
    return fp8_gemm_amd


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


@pytest.mark.parametrize("M,N,K,fa,fb", [
    (1, 16, 16, E4M3, E4M3),          # one K chunk: 3 of 4 waves idle
    (1, 4104, 7168, E4M3, E4M3),      # N tail inside a workgroup
    (16, 100, 1040, E5M2, E4M3),      # 9 K blocks, the last 16 bytes
    (17, 520, 384, E4M3, E5M2),       # two token blocks, 3 K blocks: one wave idle
    (24, 264, 4096, E4M3, E4M3),      # two token blocks, 8 steps per wave through a 3-slot ring
    (33, 264, 2048, E5M2, E5M2),      # four token blocks, 4 steps per wave through a 2-slot ring
    (64, 4096, 1024, E4M3, E4M3),
    (48, 40, 272, E4M3, E4M3),
    (1, 8200, 1040, E4M3, E4M3),      # N >= 8192: 32 weight rows per workgroup, 8-row tail
    (17, 8192, 2048, E5M2, E4M3),     # 32-row workgroups, two token blocks
    (64, 8232, 1024, E4M3, E4M3),     # 32-row workgroups, four token blocks, 8-row tail
])
def test_decode_matches_oracle(M, N, K, fa, fb):
    w = workloads.dense_random(M, N, K, seed=M * 7 + N + K, a_fmt=fa, b_fmt=fb, scales=(0.75, 1.5))
    assert _f().plan(0, M, N, K).variant == 4
    print(f"[decode] M={M} N={N} K={K} fmt=({fa},{fb})", flush=True)
    d = _f().gemm_nt(_dev(w.A), _dev(w.B), torch.tensor([w.sa], device="cuda"), torch.tensor([w.sb], device="cuda"),
                     a_dtype=fa, b_dtype=fb)
    torch.cuda.synchronize()
    d = gpu_bits(d)
    ref, r, s, _ = oracle.gemm_nt(w.A, w.B, fa, fb, w.sa, w.sb)
    check(d, r, s, abs(w.sa * w.sb), ref_bits=ref, what=f"decode {M}x{N}x{K}")


def test_decode_all_ones_exact():
    """A = B = 1.0: every output is exactly K (representable), for each token count."""
    for M in (1, 16, 17, 32, 40, 64):
        K = 2048 + 128 * (M % 3)
        A = np.full((M, K), 0x38, np.uint8)
        B = np.full((300, K), 0x38, np.uint8)
        d = _f().gemm_nt(_dev(A), _dev(B), torch.ones(1, device="cuda"), torch.ones(1, device="cuda"),
                         a_dtype=E4M3, b_dtype=E4M3)
        torch.cuda.synchronize()
        assert (d.float() == K).all(), M


@pytest.mark.parametrize("M,N,K", [(1, 300, 400), (17, 4096, 1152), (64, 520, 2000 - 2000 % 16),
                                   (33, 8200, 1152)])
def test_decode_blockscaled(M, N, K):
    w = workloads.dense_blockscaled(M, N, K, seed=M + 3 * N + K, lds_pad=5, pad_code=255)
    assert _f().plan(3, M, N, K).variant == 4
    print(f"[decode bs] M={M} N={N} K={K}", flush=True)
    d = _f().gemm_nt_blockscaled(_dev(w.A), _dev(w.B), _dev(w.sa), _dev(w.sb), a_dtype=E4M3, b_dtype=E4M3)
    torch.cuda.synchronize()
    d = gpu_bits(d)
    ref, r, s = oracle.gemm_nt_blockscaled(w.A, w.B, w.sa, w.sb)
    check(d, r, s, 1.0, ref_bits=ref, what=f"decode blockscaled {M}x{N}x{K}")


def test_decode_deterministic():
    w = workloads.dense_random(32, 4096, 7168, seed=77)
    a, b = _dev(w.A), _dev(w.B)
    one = torch.ones(1, device="cuda")
    outs = [gpu_bits(_f().gemm_nt(a, b, one, one, a_dtype=E4M3, b_dtype=E4M3)) for _ in range(3)]
    assert all(np.array_equal(outs[0], o) for o in outs[1:])
