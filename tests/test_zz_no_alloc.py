"""The allocation-free dense entry point (fp8_gemm_nt_noalloc) against
fp8_gemm_nt, through the C ABI: the same kernels, so the outputs must be
bit-identical; also within the stated bound of the oracle.

Calls in a row on the split-K few-token path (the waves-on-rows kernel, then
the waves-on-K kernel twice), each with smaller weights than the one before
and the last with fewer weight-row blocks and splits than the second (the
scratch array keeps each call's partial sums and counts, which must not leak
into the next), then a call on the tiled path (no scratch).  Collected last so that a failure here
hides no other test."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests._parity import check, gpu_bits, random_allowance

pytestmark = pytest.mark.gpu


def _f():
    import fp8_gemm_amd
    return fp8_gemm_amd


def _run(w, no_alloc):
    M, N, K = w.shape
    a = torch.from_numpy(np.ascontiguousarray(w.A)).cuda()
    b = torch.from_numpy(np.ascontiguousarray(w.B)).cuda()
    sa = torch.tensor([w.sa], dtype=torch.float32, device="cuda")
    sb = torch.tensor([w.sb], dtype=torch.float32, device="cuda")
    out = torch.full((M, N), 7.0, dtype=torch.bfloat16, device="cuda")
    _f().gemm_nt(a, b, sa, sb, out=out, a_dtype=w.a_fmt, b_dtype=w.b_fmt, no_alloc=no_alloc)
    torch.cuda.synchronize()
    return gpu_bits(out)


@pytest.mark.parametrize("order", ["noalloc_first", "alloc_first"])
def test_noalloc_matches_fp8_gemm_nt(order):
    shapes = [(64, 7168, 4096, 4), (64, 1024, 7168, 1), (20, 512, 1536, 2), (300, 520, 384, 3)]
    for M, N, K, seed in shapes:
        w = workloads.dense_random(M, N, K, seed=seed, scales=(0.75, 1.5))
        plan = _f().plan(0, M, N, K)
        print(f"[noalloc] {order} M={M} N={N} K={K} variant={plan.variant} k_splits={plan.k_splits}", flush=True)
        if order == "noalloc_first":
            d_na = _run(w, True)
            d_ref = _run(w, False)
        else:
            d_ref = _run(w, False)
            d_na = _run(w, True)
        assert np.array_equal(d_na, d_ref), f"{M}x{N}x{K}: {int((d_na != d_ref).sum())} elements differ"
        ref, r, s, _ = oracle.gemm_nt(w.A, w.B, w.a_fmt, w.b_fmt, w.sa, w.sb)
        sc = abs(w.sa * w.sb)
        check(d_na, r, s, sc, ref_bits=ref, what=f"noalloc {M}x{N}x{K}",
              **random_allowance(w.A, w.B, w.a_fmt, w.b_fmt, sc, s))
    assert _f().plan(0, 64, 1024, 7168).k_splits == 4 and _f().plan(0, 20, 512, 1536).k_splits == 3
    assert _f().plan(0, 64, 7168, 4096).tile_n == 64 and _f().plan(0, 64, 7168, 4096).k_splits == 2


def test_noalloc_needs_out():
    a = torch.zeros((4, 16), dtype=torch.uint8, device="cuda")
    one = torch.ones(1, device="cuda")
    with pytest.raises(ValueError):
        _f().gemm_nt(a, a, one, one, a_dtype=0, b_dtype=0, no_alloc=True)
