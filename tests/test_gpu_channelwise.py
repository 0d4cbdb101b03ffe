"""GPU parity of the dense FP8 GEMM with per-row / per-channel scales and a
per-channel bias (fp8_gemm_nt_channelwise) against the CPU oracle, through the
C ABI, on every shape class (decode kernel, both tiles)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests._exact import bf16_nearest_even
from tests._parity import check, gpu_bits, hw_allowance, random_cap

pytestmark = pytest.mark.gpu

E4M3, E5M2 = 0, 1


def _f():
    import fp8_gemm_amd
    return fp8_gemm_amd


def _dev(x):
    return None if x is None else torch.from_numpy(np.ascontiguousarray(x)).cuda()


def _vectors(rng, M, N, which):
    sa = rng.uniform(0.25, 2.0, M).astype(np.float32) if "a" in which else None
    sb = rng.uniform(-1.5, 1.5, N).astype(np.float32) if "b" in which else None
    bias = rng.normal(0, 20, N).astype(np.float32) if "c" in which else None
    return sa, sb, bias


def run(w, sa, sb, bias):
    M, N, K = w.shape
    print(f"[channelwise] M={M} N={N} K={K} sa={sa is not None} sb={sb is not None} bias={bias is not None}", flush=True)
    d = _f().gemm_nt_channelwise(_dev(w.A), _dev(w.B), _dev(sa), _dev(sb), _dev(bias), a_dtype=w.a_fmt, b_dtype=w.b_fmt)
    torch.cuda.synchronize()
    return gpu_bits(d)


@pytest.mark.parametrize("M,N,K,fa,fb,which", [
    (5, 130, 256, E4M3, E4M3, "abc"),       # decode kernel, N tail of 2 channels
    (17, 520, 1040, E5M2, E4M3, "bc"),
    (64, 4100, 384, E4M3, E4M3, "ac"),
    (20, 8204, 512, E4M3, E4M3, "abc"),     # decode kernel with 32-row workgroups, N tail of 12
    (300, 264, 400, E4M3, E5M2, "abc"),     # 128x256 tiles
    (513, 300, 256, E4M3, E4M3, "c"),       # 128x256 tiles, bias only
    (4000, 3800, 528, E4M3, E4M3, "abc"),   # 256x256 tiles, every edge partial, K tail
    (3968, 3840, 1024, E5M2, E4M3, "b"),    # 256x256 tiles, channel scales only
    (2000, 12000, 528, E4M3, E4M3, "abc"),  # 256x192 tiles, every edge partial, K tail
    (2000, 14000, 528, E5M2, E4M3, "abc"),  # 256x224 tiles, every edge partial, K tail
    (129, 136, 128, E5M2, E5M2, "ab"),
])
def test_channelwise_matches_oracle(M, N, K, fa, fb, which):
    rng = np.random.default_rng(M + N + K)
    w = workloads.dense_random(M, N, K, seed=M * 3 + N + K, a_fmt=fa, b_fmt=fb)
    sa, sb, bias = _vectors(rng, M, N, which)
    d = run(w, sa, sb, bias)
    ref, r, s = oracle.gemm_nt_channelwise(w.A, w.B, sa, sb, bias, fa, fb)
    # the truncation allowance per element, times that element's |sa[m] sb[n]|
    sam = np.abs(sa) if sa is not None else np.ones(M)
    sbn = np.abs(sb) if sb is not None else np.ones(N)
    _, _, s_unscaled, _ = oracle.gemm_nt(w.A, w.B, fa, fb)
    allow = hw_allowance(w.A, w.B, fa, fb, 1.0, s_unscaled) * np.outer(sam, sbn)
    check(d, r, s, 1.0, ref_bits=ref, what=f"channelwise {M}x{N}x{K} {which}", allowance=allow,
          max_allowed=random_cap(d.size, K))


def test_zero_weights_give_the_rounded_bias():
    """With B = 0 every output is bf16(bias[n]) exactly, on every kernel."""
    rng = np.random.default_rng(31)
    for M, N in [(3, 100), (200, 264), (700, 512), (3968, 3840), (2000, 12000), (2000, 14000)]:
        w = workloads.dense_random(M, N, 256, seed=31 + M)
        w.B[:] = 0
        sa, _, bias = _vectors(rng, M, N, "ac")
        d = run(w, sa, None, bias)
        want = np.array([bf16_nearest_even(float(b)) for b in bias], np.uint16)
        assert (d == want[None, :]).all(), (M, N)


def test_power_of_two_vectors_equal_per_tensor_entry_point():
    f = _f()
    for M, N in [(20, 300), (400, 520)]:
        w = workloads.dense_random(M, N, 512, seed=40 + M)
        d = run(w, np.full(M, 0.5, np.float32), np.full(N, 8.0, np.float32), None)
        d0 = f.gemm_nt(_dev(w.A), _dev(w.B), torch.tensor([0.5], device="cuda"), torch.tensor([8.0], device="cuda"),
                       a_dtype=E4M3, b_dtype=E4M3)
        torch.cuda.synchronize()
        assert np.array_equal(d, gpu_bits(d0)), (M, N)


def test_bias_cancels_sum():
    """A bias equal to minus the (exactly representable) dot product gives 0."""
    M, N, K = 4, 64, 128
    A = np.full((M, K), 0x38, np.uint8)          # 1.0
    B = np.full((N, K), 0x40, np.uint8)          # 2.0: every dot product is 256
    d = run(workloads.Dense(A, B, 1.0, 1.0), None, None, np.full(N, -256.0, np.float32))
    assert (d == 0).all()


def test_channelwise_4096_sampled():
    rng = np.random.default_rng(33)
    w = workloads.dense_square()
    sa, sb, bias = _vectors(rng, 4096, 4096, "abc")
    d = run(w, sa, sb, bias)
    ii = rng.integers(0, 4096, 1024)
    jj = rng.integers(0, 4096, 1024)
    D, R, S, _ = oracle.gemm_nt_points(w.A, w.B, ii, jj)
    sc = sa[ii].astype(np.float64) * sb[jj].astype(np.float64)
    r = R * sc + bias[jj].astype(np.float64)
    s = S * np.abs(sc)
    ref = np.array([bf16_nearest_even(float(x)) for x in r], np.uint16)
    check(d[ii, jj], r, s, 1.0, ref_bits=ref, what="channelwise 4096^3")
