"""GPU parity of the dense FP8 GEMM (fp8_gemm_nt) against the CPU oracle.

Calls go through the C ABI (via the Python binding).  Bit-exact checks where the
exact result is representable (decode table, one-hot layout, closed forms,
rounding ties); the element-wise bound of tests/_parity.py elsewhere.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests._parity import (assert_within_bound, check, gpu_bits, hw_allowance, hw_allowance_points, random_allowance,
                           random_cap)

pytestmark = pytest.mark.gpu

E4M3, E5M2 = 0, 1


def _lib():
    import fp8_gemm_amd
    return fp8_gemm_amd


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def _scale(v):
    return torch.tensor([v], dtype=torch.float32, device="cuda")


def run_dense(A, B, a_fmt, b_fmt, sa=1.0, sb=1.0, out=None):
    print(f"[dense] M={A.shape[0]} N={B.shape[0]} K={A.shape[1]} fmt=({a_fmt},{b_fmt}) sa={sa} sb={sb}", flush=True)
    f = _lib()
    d = f.gemm_nt(_dev(A), _dev(B), _scale(sa), _scale(sb), out=out, a_dtype=a_fmt, b_dtype=b_fmt)
    torch.cuda.synchronize()
    return gpu_bits(d)


def _nan_eq(a, b):
    """Bit equality, with any NaN pattern matching any NaN pattern."""
    a = np.asarray(a, np.uint16)
    b = np.asarray(b, np.uint16)
    nan_a = ((a & 0x7F80) == 0x7F80) & ((a & 0x007F) != 0)
    nan_b = ((b & 0x7F80) == 0x7F80) & ((b & 0x007F) != 0)
    return np.where(nan_a | nan_b, nan_a == nan_b, a == b)


# ---------------------------------------------------------------------------
# Bit-exact pins
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("a_fmt,b_fmt", [(E4M3, E4M3), (E5M2, E5M2), (E4M3, E5M2), (E5M2, E4M3)])
def test_decode_product_table(a_fmt, b_fmt):
    """Row i of A holds code i at k = 0, row j of B holds code j: D[i][j] is
    dec(i) * dec(j), exact in BF16, so decode and format selection are pinned
    bit for bit over all 256 x 256 code pairs."""
    K = 16
    A = np.zeros((256, K), np.uint8)
    B = np.zeros((256, K), np.uint8)
    A[:, 0] = np.arange(256)
    B[:, 0] = np.arange(256)
    ref, _, _, _ = oracle.gemm_nt(A, B, a_fmt, b_fmt)
    got = run_dense(A, B, a_fmt, b_fmt)
    ok = _nan_eq(got, ref)
    assert ok.all(), f"{int((~ok).sum())} mismatches, first at {np.argwhere(~ok)[:4].tolist()}"


@pytest.mark.parametrize("M,N,K", [(256, 256, 256), (300, 260, 384), (40, 96, 256)])
def test_one_hot_layout(M, N, K):
    """One product per output row at a distinct K position: pins the row,
    column and K placement of both operands and of the accumulator."""
    rng = np.random.default_rng(M + N + K)
    n = min(M, N, K)
    rows = rng.permutation(M)[:n]
    cols = rng.permutation(N)[:n]
    ks = rng.permutation(K)[:n]
    A = np.zeros((M, K), np.uint8)
    B = np.zeros((N, K), np.uint8)
    A[rows, ks] = 0x40      # 2.0
    B[cols, ks] = 0x48      # 4.0
    ref, _, _, _ = oracle.gemm_nt(A, B)
    got = run_dense(A, B, E4M3, E4M3)
    assert np.array_equal(got, ref)
    assert (got[rows, cols] == oracle.bf16_rne(8.0)).all()


@pytest.mark.parametrize("K", [128, 256, 1280, 4096, 7168, 14336])
@pytest.mark.parametrize("M", [48, 130])
def test_all_ones_gives_K(K, M):
    for fmt, one in ((E4M3, 0x38), (E5M2, 0x3C)):
        A = np.full((M, K), one, np.uint8)
        B = np.full((72, K), one, np.uint8)
        got = run_dense(A, B, fmt, fmt)
        assert (got == oracle.bf16_rne(float(K))).all()


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
@pytest.mark.parametrize("M", [33, 200])
def test_identity_B_returns_A(fmt, M):
    K = 256
    one = 0x38 if fmt == E4M3 else 0x3C
    rng = np.random.default_rng(5)
    codes = np.array([c for c in range(256) if np.isfinite(oracle.decode_table(fmt)[c])], np.uint8)
    A = rng.choice(codes, size=(M, K))
    B = np.zeros((K, K), np.uint8)
    np.fill_diagonal(B, one)
    ref, _, _, _ = oracle.gemm_nt(A, B, fmt, fmt)
    got = run_dense(A, B, fmt, fmt)
    # +0 and -0 compare equal
    same = (got == ref) | (((got | ref) & 0x7FFF) == 0)
    assert same.all()


def test_max_magnitude():
    K = 4096
    A = np.full((80, K), 0x7E, np.uint8)
    B = np.full((64, K), 0x7E, np.uint8)
    B[1::2] = 0xFE
    got = run_dense(A, B, E4M3, E4M3)
    assert (got[:, 0::2] == 0x4E44).all() and (got[:, 1::2] == 0xCE44).all()


def test_rounding_ties_bit_exact():
    """1 + 2^-8 -> 1.0 and 1 + 3*2^-8 -> 1 + 2^-6 (round to nearest even);
    both sums are exact in the FP32 accumulator."""
    A = np.zeros((96, 128), np.uint8)
    A[:, 0] = 0x38
    A[0::2, 1] = 0x02
    A[1::2, 1] = 0x06
    B = np.zeros((16, 128), np.uint8)
    B[:, :2] = 0x38
    got = run_dense(A, B, E4M3, E4M3)
    assert (got[0::2] == 0x3F80).all() and (got[1::2] == 0x3F82).all()


def test_power_of_two_scale_is_exact():
    w = workloads.dense_random(130, 96, 512, seed=17)
    d1 = run_dense(w.A, w.B, E4M3, E4M3, 1.0, 1.0)
    d4 = run_dense(w.A, w.B, E4M3, E4M3, 2.0, 2.0)
    x1 = torch.from_numpy(d1.view(np.int16)).view(torch.bfloat16).float()
    x4 = torch.from_numpy(d4.view(np.int16)).view(torch.bfloat16).float()
    assert torch.equal(x1 * 4, x4)


# ---------------------------------------------------------------------------
# Bound checks
# ---------------------------------------------------------------------------

def _check_dense(w, what, out=None, seeded=False):
    """Random inputs take the capped truncation allowance; the seeded
    configurations the stated bound alone."""
    d = run_dense(w.A, w.B, w.a_fmt, w.b_fmt, w.sa, w.sb, out=out)
    ref, r, s, _ = oracle.gemm_nt(w.A, w.B, w.a_fmt, w.b_fmt, w.sa, w.sb)
    sc = abs(w.sa * w.sb)
    extra = {} if seeded else random_allowance(w.A, w.B, w.a_fmt, w.b_fmt, sc, s)
    check(d, r, s, sc, ref_bits=ref, what=what, **extra)
    return d


# (64 x 65 x 16 has 1 element that needs the allowance on the GPU.)
SHAPES = [(1, 1, 16), (1, 200, 128), (7, 64, 144), (16, 257, 112), (17, 129, 1280), (33, 255, 256),
          (63, 64, 128), (64, 65, 16), (65, 64, 128), (127, 128, 144), (128, 127, 256), (129, 257, 384),
          (255, 300, 640), (257, 255, 1280), (300, 520, 272), (513, 260, 128)]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_ragged_shapes_e4m3(M, N, K):
    w = workloads.dense_random(M, N, K, seed=M * 7 + N * 3 + K, std=1.0, scales=(0.75, 1.5))
    _check_dense(w, f"{M}x{N}x{K}")


@pytest.mark.parametrize("a_fmt,b_fmt", [(E5M2, E5M2), (E4M3, E5M2), (E5M2, E4M3)])
@pytest.mark.parametrize("M,N,K", [(40, 136, 384), (300, 264, 512)])
def test_formats(M, N, K, a_fmt, b_fmt):
    w = workloads.dense_random(M, N, K, seed=99, a_fmt=a_fmt, b_fmt=b_fmt, scales=(1.25, 0.5))
    _check_dense(w, f"{M}x{N}x{K} fmt {a_fmt}{b_fmt}")


def test_dense_256_config():
    """Seeded 256^3 configuration: the stated bound on every element."""
    w = workloads.dense_small()
    _check_dense(w, "dense 256^3", seeded=True)


def test_built_cancelling_sums():
    """Where a sum cancels (|r| far below S) the matrix cores' truncation of
    products to the largest product's exponent in each group of 8 K indices
    (tests/test_gpu_mfma_numerics.py) is the whole error, and the stated bound's
    2^-8 |r| term no longer covers it.  This input is built to cancel, so it
    passes the allowance H + F explicitly, with no cap on the count; every
    element outside the stated bound must lie within it plus the allowance.  130 x 72 x 32 (tiled kernel): K indices 16..31 repeat 0..15 of
    A with one code step changed in a random half, against the negated B, so
    each sum is a few code steps of A times B (a CPU model of the measured rule
    puts 1153 of the 9360 sums outside the stated bound)."""
    rng = np.random.default_rng(1616)
    M, N, K = 130, 72, 32
    codes = np.arange(1, 0x7E, dtype=np.uint8)      # positive finite E4M3 values, no zero
    A = np.zeros((M, K), np.uint8)
    B = np.zeros((N, K), np.uint8)
    A[:, :16] = rng.choice(codes, size=(M, 16))
    step = rng.integers(0, 2, size=(M, 16)) * rng.choice([-1, 1], size=(M, 16))
    A[:, 16:] = np.clip(A[:, :16].astype(np.int64) + step, 1, 0x7D).astype(np.uint8)
    B[:, :16] = rng.choice(codes, size=(N, 16))
    B[:, 16:] = B[:, :16] | 0x80                    # the negated values
    d = run_dense(A, B, E4M3, E4M3)
    ref, r, s, _ = oracle.gemm_nt(A, B)
    check(d, r, s, 1.0, ref_bits=ref, what="130x72x32 built to cancel",
          allowance=hw_allowance(A, B, E4M3, E4M3, 1.0, s), max_allowed=M * N)


def test_strided_operands_and_output():
    M, N, K = 200, 136, 256
    w = workloads.dense_random(M, N, K, seed=12)
    A = np.zeros((M, K + 48), np.uint8)
    A[:, :K] = w.A
    B = np.zeros((N, K + 16), np.uint8)
    B[:, :K] = w.B
    f = _lib()
    a = _dev(A)[:, :K]
    b = _dev(B)[:, :K]
    big = torch.full((M, N + 40), -7.0, dtype=torch.bfloat16, device="cuda")
    out = big[:, :N]
    f.gemm_nt(a, b, _scale(1.0), _scale(1.0), out=out, a_dtype=E4M3, b_dtype=E4M3)
    torch.cuda.synchronize()
    ref, r, s, _ = oracle.gemm_nt(w.A, w.B)
    check(gpu_bits(out), r, s, 1.0, ref_bits=ref, what="strided", **random_allowance(w.A, w.B, E4M3, E4M3, 1.0, s))
    assert (big[:, N:] == -7.0).all()


def _sample_points(M, N, n, seed):
    rng = np.random.default_rng(seed)
    ii = np.concatenate([rng.integers(0, M, n), np.zeros(N // 8, np.int64), np.full(N // 8, M - 1)])
    jj = np.concatenate([rng.integers(0, N, n), np.arange(0, N, 8), np.arange(3, N, 8)])
    return ii, jj


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_dense_4096_config_sampled(fmt):
    w = workloads.dense_square(fmt)
    M, N, K = w.shape
    d = run_dense(w.A, w.B, fmt, fmt, w.sa, w.sb)
    ii, jj = _sample_points(M, N, 6000, seed=fmt)
    ref, r, s, ex = oracle.gemm_nt_points(w.A, w.B, ii, jj, fmt, fmt, w.sa, w.sb, want_exact=True)
    # the oracle's FP64 sums are exact here (its integer cross-check agrees),
    # so r is the exact scaled sum rounded once
    assert (ex == 1).all(), f"{int((ex != 1).sum())} sampled sums not exact in FP64"
    # seeded configuration: the stated bound on every checked element
    assert_within_bound(d[ii, jj], r, s, abs(w.sa * w.sb), ref_bits=ref, what=f"4096^3 fmt {fmt}")
    # full rows through the tile boundaries
    rows = np.array([0, 255, 256, 4095])
    Dr, Rr, Sr, _ = oracle.gemm_nt(w.A[rows], w.B, fmt, fmt, w.sa, w.sb)
    assert_within_bound(d[rows], Rr, Sr, abs(w.sa * w.sb), ref_bits=Dr, what="full rows")


# The tile class the planner picks for each transformer-projection shape
# (1 = 256x256, 2 = 128x256, 5 = 256x192, 6 = 256x224): whole waves of 256
# workgroups wherever a class gives them.
PROJECTION_VARIANTS = {
    (2048, 4096, 4096): 2, (2048, 14336, 4096): 6, (2048, 4096, 14336): 2, (2048, 12288, 4096): 5,
    (8192, 4096, 4096): 1, (8192, 14336, 4096): 1, (8192, 4096, 14336): 1, (8192, 12288, 4096): 1,
}


@pytest.mark.parametrize("idx", range(len(workloads.PROJECTION_SHAPES)))
def test_projection_configs_sampled(idx):
    """The eight seeded transformer-projection configurations (E4M3
    activations N(0,1), amax-scaled N(0, 0.02) weights, K up to 14336, 8192-row
    shapes) in the tile class the planner picks for them, against the stated
    bound alone: 4000 random points plus full rows on both sides of the first
    tile boundary and the last row, with the oracle's FP64 sums exact."""
    w = workloads.projection(idx)
    M, N, K = w.shape
    plan = _lib().plan(0, M, N, K)
    assert plan.variant == PROJECTION_VARIANTS[(M, N, K)], plan.variant
    d = run_dense(w.A, w.B, w.a_fmt, w.b_fmt, w.sa, w.sb)
    ii, jj = _sample_points(M, N, 4000, seed=30 + idx)
    ref, r, s, ex = oracle.gemm_nt_points(w.A, w.B, ii, jj, w.a_fmt, w.b_fmt, w.sa, w.sb, want_exact=True)
    assert (ex == 1).all()
    assert_within_bound(d[ii, jj], r, s, abs(w.sa * w.sb), ref_bits=ref, what=f"projection {M}x{N}x{K} sampled")
    tm = plan.tile_m
    rows = np.array([0, tm - 1, tm, M - 1])
    Dr, Rr, Sr, _ = oracle.gemm_nt(w.A[rows], w.B, w.a_fmt, w.b_fmt, w.sa, w.sb)
    assert_within_bound(d[rows], Rr, Sr, abs(w.sa * w.sb), ref_bits=Dr, what=f"projection {M}x{N}x{K} rows {rows.tolist()}")


@pytest.mark.parametrize("M,N,K,fa,fb", [
    (4000, 3800, 528, E4M3, E4M3),      # M, N and K tails (K = 4 * 128 + 16)
    (3900, 3800, 1040, E5M2, E4M3),     # K = 8 * 128 + 16
    (4000, 3800, 1024, E4M3, E5M2),     # M and N tails only
    (3968, 3840, 272, E5M2, E5M2),
    (3968, 3840, 16, E4M3, E4M3),       # one partial K step (the ring's second slot only prefetches)
    (4000, 3800, 144, E4M3, E5M2),      # two steps, the second partial
])
def test_256_tiles_ragged_full(M, N, K, fa, fb):
    """The 256 x 256-tile kernel (the plan picks it for these shapes) with
    partial tiles on every edge, every format pair and K tails of 16 bytes:
    the whole output against the oracle."""
    assert _lib().plan(0, M, N, K).variant == 1
    w = workloads.dense_random(M, N, K, seed=M + N + K, a_fmt=fa, b_fmt=fb, std=1.0, scales=(0.5, 1.5))
    _check_dense(w, f"256-tile {M}x{N}x{K} fmt ({fa},{fb})")


@pytest.mark.parametrize("M,N,K,fa,fb", [
    (2000, 12000, 1040, E4M3, E4M3),    # 256 x 192 tiles: partial tiles on both edges, K tail
    (1900, 11600, 528, E5M2, E4M3),
])
def test_256x192_tiles_full(M, N, K, fa, fb):
    """The 256 x 192 tiles (picked where whole waves of them replace a partial
    wave of 256 x 256 tiles): the whole output against the oracle."""
    assert _lib().plan(0, M, N, K).variant == 5
    w = workloads.dense_random(M, N, K, seed=M + N + K, a_fmt=fa, b_fmt=fb, std=1.0, scales=(0.5, 1.5))
    _check_dense(w, f"256x192-tile {M}x{N}x{K} fmt ({fa},{fb})")


@pytest.mark.parametrize("M,N,K,fa,fb", [
    (2000, 14000, 1040, E4M3, E4M3),    # 256 x 224 tiles: partial tiles on both edges, K tail
    (1900, 13900, 528, E5M2, E4M3),
    (2000, 14000, 144, E5M2, E5M2),     # second K step partial
    (2048, 14336, 384, E4M3, E5M2),     # whole tiles, no K tail
])
def test_256x224_tiles_full(M, N, K, fa, fb):
    """The 256 x 224 tiles (7 weight blocks per wave, an odd number of B
    copies per wave, so the K-tail key parity flips with the wave): the whole
    output against the oracle."""
    assert _lib().plan(0, M, N, K).variant == 6
    w = workloads.dense_random(M, N, K, seed=M + N + K, a_fmt=fa, b_fmt=fb, std=1.0, scales=(0.5, 1.5))
    _check_dense(w, f"256x224-tile {M}x{N}x{K} fmt ({fa},{fb})")


@pytest.mark.parametrize("M,N,K", [(6144, 6144, 1280), (4096, 4096, 1024)])
def test_k_tail_regression_shapes_sampled(M, N, K):
    """Shapes from "DeepGEMM on Hopper Tensor Cores", section 6.1: one failed
    there (K=1280), one passed (K=1024)."""
    w = workloads.dense_random(M, N, K, seed=61, std=0.5, scales=(1.0, 1.0))
    d = run_dense(w.A, w.B, E4M3, E4M3)
    ii, jj = _sample_points(M, N, 4000, seed=K)
    ref, r, s, _ = oracle.gemm_nt_points(w.A, w.B, ii, jj)
    check(d[ii, jj], r, s, 1.0, ref_bits=ref, what=f"{M}x{N}x{K}",
          allowance=hw_allowance_points(w.A, w.B, ii, jj, E4M3, E4M3, 1.0, s), max_allowed=random_cap(len(ii), K))


# Seeded random shapes (M 65..4096, N 16..16384, K a multiple of 16 up to
# 2048, random formats), three for each tile class the planner picks: the
# plan is the recorded one (tile class, workgroups) and every output matches
# the oracle.
@pytest.mark.parametrize("M,N,K,a_fmt,b_fmt,variant,workgroups", [
    (2155, 7030, 576, 1, 0, 1, 252), (3804, 4201, 400, 1, 1, 1, 255), (1432, 9417, 560, 1, 0, 1, 222),
    (154, 6359, 1904, 1, 1, 2, 50), (1688, 3972, 1184, 1, 1, 2, 224), (2075, 1076, 80, 1, 1, 2, 85),
    (1019, 8752, 1328, 0, 0, 5, 184), (2223, 4482, 1056, 0, 0, 5, 216), (722, 11269, 1120, 1, 0, 5, 177),
    (2485, 10412, 384, 0, 0, 6, 470), (3354, 11734, 176, 1, 1, 6, 742), (1844, 13866, 48, 1, 1, 6, 496),
])
def test_tiled_random_shapes(M, N, K, a_fmt, b_fmt, variant, workgroups):
    plan = _lib().plan(0, M, N, K)
    assert (plan.variant, plan.workgroups) == (variant, workgroups)
    w = workloads.dense_random(M, N, K, seed=M + N + K, a_fmt=a_fmt, b_fmt=b_fmt, scales=(0.5, 1.25))
    _check_dense(w, f"random {M}x{N}x{K} fmt ({a_fmt},{b_fmt}) variant {variant}")


def test_deterministic_repeats():
    w = workloads.dense_random(512, 384, 1024, seed=3)
    outs = [run_dense(w.A, w.B, E4M3, E4M3) for _ in range(3)]
    assert all(np.array_equal(outs[0], o) for o in outs[1:])
    ws = workloads.dense_random(24, 384, 1024, seed=4)
    outs = [run_dense(ws.A, ws.B, E4M3, E4M3) for _ in range(3)]
    assert all(np.array_equal(outs[0], o) for o in outs[1:])


@pytest.mark.parametrize("M,N", [(48, 300), (300, 48)])
def test_swap_identity(M, N):
    """D^T = B . A^T: the swapped call (which may take the other kernel) is
    within the bound of the transposed oracle result."""
    K = 768
    w = workloads.dense_random(M, N, K, seed=8)
    dt = run_dense(w.B, w.A, E4M3, E4M3)
    ref, r, s, _ = oracle.gemm_nt(w.A, w.B)
    check(dt.T, r, s, 1.0, ref_bits=ref, what="swap identity", **random_allowance(w.A, w.B, E4M3, E4M3, 1.0, s))


def test_nan_inputs_propagate():
    M, N, K = 100, 80, 256
    w = workloads.dense_random(M, N, K, seed=10)
    A = w.A.copy()
    B = w.B.copy()
    A[5, 17] = 0x7F
    B[9, 200] = 0x7F
    d = run_dense(A, B, E4M3, E4M3)
    ref, r, s, _ = oracle.gemm_nt(A, B)
    check(d, r, s, 1.0, ref_bits=ref, what="nan inputs", **random_allowance(A, B, E4M3, E4M3, 1.0, s))


def test_zero_sizes_and_empty_k():
    f = _lib()
    a = torch.zeros((0, 32), dtype=torch.uint8, device="cuda")
    b = torch.zeros((16, 32), dtype=torch.uint8, device="cuda")
    out = f.gemm_nt(a, b, _scale(1.0), _scale(1.0), a_dtype=E4M3, b_dtype=E4M3)
    assert out.shape == (0, 16)
    a = torch.zeros((70, 0), dtype=torch.uint8, device="cuda")
    b = torch.zeros((24, 0), dtype=torch.uint8, device="cuda")
    out = torch.full((70, 24), 3.0, dtype=torch.bfloat16, device="cuda")
    f.gemm_nt(a, b, _scale(1.0), _scale(1.0), out=out, a_dtype=E4M3, b_dtype=E4M3)
    torch.cuda.synchronize()
    assert (out == 0).all()


def test_validation_errors_through_binding():
    f = _lib()
    a = torch.zeros((64, 40), dtype=torch.uint8, device="cuda")   # K = 40: not a multiple of 16
    b = torch.zeros((64, 40), dtype=torch.uint8, device="cuda")
    with pytest.raises(f.Fp8GemmError) as e:
        f.gemm_nt(a, b, _scale(1.0), _scale(1.0), a_dtype=E4M3, b_dtype=E4M3)
    assert e.value.status == -2
