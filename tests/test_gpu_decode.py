"""GPU parity of the dense few-token (M <= 64) path, the swap-AB decode kernels
(K split over 4 waves with per-wave LDS rings, or the 4 waves on 16 weight
rows each sharing the token copies) against the CPU oracle, through the C ABI.

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
from tests._parity import check, gpu_bits, hw_allowance, hw_allowance_blockscaled, random_allowance, random_cap

pytestmark = pytest.mark.gpu

E4M3, E5M2 = 0, 1


def _f():
    import fp8_gemm_amd
    return fp8_gemm_amd


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


# K splits (workgroups per block of weight rows) these take: (16, 100, 1040)
# 2 (5 + 4 K steps), (24, 264, 4096) 8, (33, 264, 2048) 4, (64, 1000, 1536)
# 3 with an 8-row last block, (40, 2056, 7168) 2 (28 steps each, 8-row last
# block); the others 1.
@pytest.mark.parametrize("M,N,K,fa,fb", [
    (1, 16, 16, E4M3, E4M3),          # one K chunk: 3 of 4 waves idle
    (1, 4104, 7168, E4M3, E4M3),      # N tail inside a workgroup
    (16, 100, 1040, E5M2, E4M3),      # 9 K blocks, the last 16 bytes
    (17, 520, 384, E4M3, E5M2),       # two token blocks, 3 K blocks: one wave idle
    (24, 264, 4096, E4M3, E4M3),      # two token blocks, 8 steps per wave through a 3-slot ring
    (33, 264, 2048, E5M2, E5M2),      # four token blocks, 4 steps per wave through a 2-slot ring
    (64, 4096, 1024, E4M3, E4M3),
    (48, 40, 272, E4M3, E4M3),
    (64, 1000, 1536, E4M3, E4M3),
    (40, 2056, 7168, E5M2, E4M3),
    (1, 8200, 1040, E4M3, E4M3),      # N >= 8192: 32 weight rows per workgroup, 8-row tail
    (17, 8192, 2048, E5M2, E4M3),     # 32-row workgroups, two token blocks
    (64, 8232, 1024, E4M3, E4M3),     # 32-row workgroups, four token blocks, 8-row tail
])
def test_decode_matches_oracle(M, N, K, fa, fb):
    w = workloads.dense_random(M, N, K, seed=M * 7 + N + K, a_fmt=fa, b_fmt=fb, scales=(0.75, 1.5))
    plan = _f().plan(0, M, N, K)
    assert plan.variant == 4
    print(f"[decode] M={M} N={N} K={K} fmt=({fa},{fb}) rows/wg={plan.tile_n} k_splits={plan.k_splits}", flush=True)
    d = _f().gemm_nt(_dev(w.A), _dev(w.B), torch.tensor([w.sa], device="cuda"), torch.tensor([w.sb], device="cuda"),
                     a_dtype=fa, b_dtype=fb)
    torch.cuda.synchronize()
    d = gpu_bits(d)
    ref, r, s, _ = oracle.gemm_nt(w.A, w.B, fa, fb, w.sa, w.sb)
    sc = abs(w.sa * w.sb)
    check(d, r, s, sc, ref_bits=ref, what=f"decode {M}x{N}x{K}", **random_allowance(w.A, w.B, fa, fb, sc, s))


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
    check(d, r, s, 1.0, ref_bits=ref, what=f"decode blockscaled {M}x{N}x{K}",
          allowance=hw_allowance_blockscaled(w.A, w.B, 0, 0, w.sa, w.sb, s), max_allowed=random_cap(d.size, K))


@pytest.mark.parametrize("M,N,K,fa,fb", [
    (1, 4104, 7168, E4M3, E4M3),      # 3 splits of 19/19/18 steps; last block 8 rows (3 waves without rows); padding column
    (37, 7160, 4000, E5M2, E4M3),     # 2 splits, K tail of 32 bytes, last block 56 rows
    (16, 10240, 2048, E4M3, E5M2),    # one token block, K not split (160 workgroups)
    (32, 14336, 4096, E4M3, E4M3),    # two token blocks, K not split (224 workgroups)
    (64, 5120, 7168, E5M2, E5M2),     # 3 splits of 19/19/18 steps, four token blocks
    (20, 7168, 4096, E4M3, E4M3),     # 2 splits, two token blocks
])
def test_decode_rows_matches_oracle(M, N, K, fa, fb):
    """The waves-on-rows few-token kernel (64 weight rows per workgroup, the 4
    waves on 16 rows each, one shared copy of the tokens per K step): the
    per-tensor, per-channel and block-scaled forms against the oracle, over
    ragged M, N and K, split and unsplit."""
    f = _f()
    plan = f.plan(0, M, N, K)
    assert plan.variant == 4 and plan.tile_n == 64 and f.plan(3, M, N, K).tile_n == 64
    print(f"[decode rows] M={M} N={N} K={K} fmt=({fa},{fb}) k_splits={plan.k_splits} workgroups={plan.workgroups}",
          flush=True)
    w = workloads.dense_random(M, N, K, seed=M * 5 + N + K, a_fmt=fa, b_fmt=fb, scales=(0.75, 1.5))
    d = gpu_bits(f.gemm_nt(_dev(w.A), _dev(w.B), torch.tensor([w.sa], device="cuda"), torch.tensor([w.sb], device="cuda"),
                           a_dtype=fa, b_dtype=fb))
    ref, r, s, _ = oracle.gemm_nt(w.A, w.B, fa, fb, w.sa, w.sb)
    sc = abs(w.sa * w.sb)
    check(d, r, s, sc, ref_bits=ref, what=f"decode rows {M}x{N}x{K}", **random_allowance(w.A, w.B, fa, fb, sc, s))
    rng = np.random.default_rng(M + N)
    csa = rng.uniform(0.5, 2, M).astype(np.float32)
    csb = rng.uniform(0.5, 2, N).astype(np.float32)
    bias = rng.normal(0, 4, N).astype(np.float32)
    d = gpu_bits(f.gemm_nt_channelwise(_dev(w.A), _dev(w.B), _dev(csa), _dev(csb), _dev(bias), a_dtype=fa, b_dtype=fb))
    ref, r, s = oracle.gemm_nt_channelwise(w.A, w.B, csa, csb, bias, fa, fb)
    _, _, s1, _ = oracle.gemm_nt(w.A, w.B, fa, fb)
    allow = hw_allowance(w.A, w.B, fa, fb, 1.0, s1) * np.outer(csa, csb)
    check(d, r, s, 1.0, ref_bits=ref, what=f"decode rows channelwise {M}x{N}x{K}", allowance=allow,
          max_allowed=random_cap(d.size, K))
    wb = workloads.dense_blockscaled(M, N, K, seed=M + 2 * N + K, lds_pad=5, pad_code=255)
    d = gpu_bits(f.gemm_nt_blockscaled(_dev(wb.A), _dev(wb.B), _dev(wb.sa), _dev(wb.sb), a_dtype=E4M3, b_dtype=E4M3))
    ref, r, s = oracle.gemm_nt_blockscaled(wb.A, wb.B, wb.sa, wb.sb)
    check(d, r, s, 1.0, ref_bits=ref, what=f"decode rows blockscaled {M}x{N}x{K}",
          allowance=hw_allowance_blockscaled(wb.A, wb.B, 0, 0, wb.sa, wb.sb, s), max_allowed=random_cap(d.size, K))


@pytest.mark.parametrize("M,N,K,rows", [
    (1, 4096, 7168, 16), (16, 4096, 7168, 16), (32, 4096, 7168, 16), (64, 4096, 7168, 16),
    (1, 14336, 4096, 64), (16, 14336, 4096, 64), (32, 14336, 4096, 64), (64, 14336, 4096, 64),
    (1, 2048, 7168, 16), (64, 2048, 7168, 16),
])
def test_bench_decode_shapes_full(M, N, K, rows):
    """Every few-token shape the benchmark times, with its inputs (A and B
    ~N(0,1) E4M3, seed 13) and in its launch configuration (the plan's kernel
    and K splits), every output against the oracle under the stated bound."""
    f = _f()
    plan = f.plan(0, M, N, K)
    assert plan.variant == 4 and plan.tile_n == rows
    print(f"[bench decode] M={M} N={N} K={K} rows/wg={plan.tile_n} k_splits={plan.k_splits}", flush=True)
    w = workloads.dense_random(M, N, K, seed=13, std=1.0)
    one = torch.ones(1, device="cuda")
    d = gpu_bits(f.gemm_nt(_dev(w.A), _dev(w.B), one, one, a_dtype=w.a_fmt, b_dtype=w.b_fmt))
    ref, r, s, _ = oracle.gemm_nt(w.A, w.B, w.a_fmt, w.b_fmt)
    check(d, r, s, 1.0, ref_bits=ref, what=f"bench decode {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K,rows", [(40, 1000, 2048, 16), (37, 7160, 4000, 64), (16, 10240, 2048, 64), (64, 8232, 1024, 32)])
def test_decode_strided_operands_and_output(M, N, K, rows):
    """Both few-token kernels (split and unsplit) with row strides above K
    for A and B and above N for D: the outputs match the oracle and the
    padding columns of D keep their sentinel."""
    f = _f()
    assert f.plan(0, M, N, K).tile_n == rows
    print(f"[decode strided] M={M} N={N} K={K} rows/wg={rows}", flush=True)
    w = workloads.dense_random(M, N, K, seed=M + N + K + 1)
    A = np.zeros((M, K + 48), np.uint8)
    A[:, :K] = w.A
    B = np.zeros((N, K + 16), np.uint8)
    B[:, :K] = w.B
    a = _dev(A)[:, :K]
    b = _dev(B)[:, :K]
    big = torch.full((M, N + 40), -7.0, dtype=torch.bfloat16, device="cuda")
    out = big[:, :N]
    one = torch.ones(1, device="cuda")
    f.gemm_nt(a, b, one, one, out=out, a_dtype=E4M3, b_dtype=E4M3)
    torch.cuda.synchronize()
    ref, r, s, _ = oracle.gemm_nt(w.A, w.B)
    check(gpu_bits(out), r, s, 1.0, ref_bits=ref, what=f"decode strided {M}x{N}x{K}",
          **random_allowance(w.A, w.B, E4M3, E4M3, 1.0, s))
    assert (big[:, N:] == -7.0).all()


# Drawn once with numpy's default_rng(2024): M in [1, 64], N in [4000, 15500),
# K a multiple of 16 in [1920, 8320); the plan's rows per workgroup and K
# splits recorded beside each (waves on rows for 9 of the 14).
@pytest.mark.parametrize("M,N,K,rows,splits", [
    (16, 11772, 2496, 64, 1), (14, 7652, 3888, 16, 1), (59, 13193, 7776, 64, 1), (64, 4903, 2816, 16, 1),
    (56, 4905, 2976, 16, 1), (12, 14508, 4208, 64, 2), (17, 5950, 4848, 64, 2), (38, 13202, 5856, 64, 1),
    (64, 5211, 5040, 64, 2), (37, 11906, 1936, 64, 1), (13, 9348, 2336, 32, 1), (63, 11377, 7024, 64, 1),
    (33, 10863, 4128, 64, 1), (21, 5490, 3232, 16, 1),
])
def test_decode_random_shapes(M, N, K, rows, splits):
    """Random few-token shapes around the plan's boundaries between the two
    kernels (ragged M, N and K): the plan is the recorded one and every output
    matches the oracle."""
    f = _f()
    plan = f.plan(0, M, N, K)
    assert (plan.tile_n, plan.k_splits) == (rows, splits)
    print(f"[decode random] M={M} N={N} K={K} rows/wg={rows} k_splits={splits}", flush=True)
    w = workloads.dense_random(M, N, K, seed=N + K, scales=(0.5, 1.25))
    d = gpu_bits(f.gemm_nt(_dev(w.A), _dev(w.B), torch.tensor([w.sa], device="cuda"), torch.tensor([w.sb], device="cuda"),
                           a_dtype=w.a_fmt, b_dtype=w.b_fmt))
    ref, r, s, _ = oracle.gemm_nt(w.A, w.B, w.a_fmt, w.b_fmt, w.sa, w.sb)
    sc = abs(w.sa * w.sb)
    check(d, r, s, sc, ref_bits=ref, what=f"decode random {M}x{N}x{K}", **random_allowance(w.A, w.B, w.a_fmt, w.b_fmt, sc, s))


_FIRST_CALL_CAPTURED = r"""
import sys
sys.path.insert(0, sys.argv[1])
import numpy as np, torch
import fp8_gemm_amd as f, oracle, workloads
from tests._parity import check, gpu_bits, random_allowance
M, N, K = 64, 7168, 4096
plan = f.plan(0, M, N, K)
assert plan.tile_n == 64 and plan.k_splits == 2, (plan.tile_n, plan.k_splits)
w = workloads.dense_random(M, N, K, seed=93)
a = torch.from_numpy(w.A).cuda()
b = torch.from_numpy(w.B).cuda()
one = torch.ones(1, device="cuda")
out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
torch.cuda.synchronize()
g = torch.cuda.CUDAGraph()
with torch.cuda.graph(g):
    f.gemm_nt(a, b, one, one, out=out, a_dtype=0, b_dtype=0)
ref, r, s, _ = oracle.gemm_nt(w.A, w.B)
allow = random_allowance(w.A, w.B, 0, 0, 1.0, s)
for i in range(2):
    out.fill_(7.0)
    g.replay()
    torch.cuda.synchronize()
    check(gpu_bits(out), r, s, 1.0, ref_bits=ref, what=f"captured first call, replay {i}", **allow)
eager = gpu_bits(f.gemm_nt(a, b, one, one, a_dtype=0, b_dtype=0))
check(eager, r, s, 1.0, ref_bits=ref, what="eager call after the capture", **allow)
print("ok")
"""


def test_split_k_first_call_under_capture():
    """In a fresh process, the first call of a shape that splits K is captured
    into a graph: the library allocates nothing during capture and runs that
    call unsplit, so the replays are correct (within the bound), and the
    eager call after it (which allocates the workspace and splits) is too."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    print("[capture first call] M=64 N=7168 K=4096 in a subprocess", flush=True)
    res = subprocess.run([sys.executable, "-c", _FIRST_CALL_CAPTURED, root], cwd=root, capture_output=True,
                         text=True, timeout=240)
    assert res.returncode == 0 and res.stdout.strip().endswith("ok"), res.stdout[-2000:] + res.stderr[-4000:]


def test_decode_deterministic():
    w = workloads.dense_random(32, 4096, 7168, seed=77)
    a, b = _dev(w.A), _dev(w.B)
    one = torch.ones(1, device="cuda")
    outs = [gpu_bits(_f().gemm_nt(a, b, one, one, a_dtype=E4M3, b_dtype=E4M3)) for _ in range(3)]
    assert all(np.array_equal(outs[0], o) for o in outs[1:])


@pytest.mark.parametrize("M,N,K,rows", [(64, 1024, 7168, 16), (64, 7168, 4096, 64)])
def test_decode_split_k_graph_replays(M, N, K, rows):
    """The split-K few-token path (both kernels: waves on K, 16 rows per
    workgroup, and waves on rows, 64) captured in a graph and replayed four
    times, with eager launches (another split shape, a fill) between the
    replays: every replay equals the eager result bit for bit, so the arrival
    counts are back at zero after each launch and the partial sums are added
    in the same order whichever split finishes last."""
    f = _f()
    w = workloads.dense_random(M, N, K, seed=91)
    w2 = workloads.dense_random(33, 1000, 2048, seed=92)
    plan = f.plan(0, M, N, K)
    assert plan.k_splits > 1 and plan.tile_n == rows and f.plan(0, 33, 1000, 2048).k_splits > 1
    a, b = _dev(w.A), _dev(w.B)
    a2, b2 = _dev(w2.A), _dev(w2.B)
    one = torch.ones(1, device="cuda")
    eager = gpu_bits(f.gemm_nt(a, b, one, one, a_dtype=E4M3, b_dtype=E4M3))
    eager2 = gpu_bits(f.gemm_nt(a2, b2, one, one, a_dtype=E4M3, b_dtype=E4M3))
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        f.gemm_nt(a, b, one, one, out=out, a_dtype=E4M3, b_dtype=E4M3)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        f.gemm_nt(a, b, one, one, out=out, a_dtype=E4M3, b_dtype=E4M3)
    for i in range(4):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(gpu_bits(out), eager), f"replay {i}"
        d2 = gpu_bits(f.gemm_nt(a2, b2, one, one, a_dtype=E4M3, b_dtype=E4M3))
        torch.cuda.synchronize()
        assert np.array_equal(d2, eager2), f"eager call after replay {i}"
    del g
    ref, r, s, _ = oracle.gemm_nt(w.A, w.B)
    check(eager, r, s, 1.0, ref_bits=ref, what=f"split-K {M}x{N}x{K}", **random_allowance(w.A, w.B, E4M3, E4M3, 1.0, s))


@pytest.mark.parametrize("M,N,K", [(64, 1024, 7168), (17, 1000, 2048), (40, 2056, 7168),
                                   (64, 7168, 4096), (1, 14336, 4096), (1, 4104, 7168)])
def test_decode_split_k_repeats(M, N, K):
    """50 launches in a row of one split shape, alternating two output
    buffers: every result equals the first bit for bit, and the first is
    within the bound of the oracle.  All splits of a block meet in one XCD's
    L2 (workgroups (x, y) with x a multiple of 8 apart go to the same XCD);
    were a split's partial sums not yet visible to the last one, some launch
    would differ.  (1000 rows: 63 blocks, a padding column of workgroups;
    2056 rows: 129 blocks, a grid above 256 workgroups, two per CU; the last
    three take the waves-on-rows kernel: 2 splits of 112 blocks, 2 splits of
    224 blocks over 448 workgroups, 3 splits of 65 blocks with a padding
    column.)"""
    f = _f()
    plan = f.plan(0, M, N, K)
    assert plan.k_splits > 1 and plan.workgroups % 8 == 0
    print(f"[split repeats] M={M} N={N} K={K} k_splits={plan.k_splits} workgroups={plan.workgroups}", flush=True)
    w = workloads.dense_random(M, N, K, seed=M + N + K)
    a, b = _dev(w.A), _dev(w.B)
    one = torch.ones(1, device="cuda")
    outs = [torch.empty((M, N), dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    first = None
    for i in range(50):
        o = outs[i % 2]
        o.fill_(7.0)
        f.gemm_nt(a, b, one, one, out=o, a_dtype=E4M3, b_dtype=E4M3)
        torch.cuda.synchronize()
        d = gpu_bits(o)
        if first is None:
            first = d
        else:
            assert np.array_equal(d, first), f"launch {i} differs in {int((d != first).sum())} elements"
    ref, r, s, _ = oracle.gemm_nt(w.A, w.B)
    check(first, r, s, 1.0, ref_bits=ref, what=f"split-K {M}x{N}x{K}", **random_allowance(w.A, w.B, E4M3, E4M3, 1.0, s))


@pytest.mark.parametrize("M,N,K,fa,fb", [
    (65, 64, 128, E4M3, E4M3),        # two token tiles, the second of 1 row
    (200, 100, 1040, E5M2, E4M3),     # 4 token tiles (the last 8 rows), N tail, K tail
    (256, 256, 256, E4M3, E5M2),      # the 256^3 shape: 16 x 4 workgroups
])
def test_small_class_token_tiles(M, N, K, fa, fb):
    """Small problems (M <= 256 where the tiled kernel would start at most 2
    workgroups) run the decode kernel over 64-token tiles: per-tensor,
    per-channel and block-scaled forms against the oracle."""
    f = _f()
    plan = f.plan(0, M, N, K)
    assert plan.variant == 4 and plan.tile_m == 64 and f.plan(3, M, N, K).variant == 4
    print(f"[small] M={M} N={N} K={K} fmt=({fa},{fb}) workgroups={plan.workgroups}", flush=True)
    w = workloads.dense_random(M, N, K, seed=M + N + K, a_fmt=fa, b_fmt=fb, scales=(0.75, 1.5))
    d = gpu_bits(f.gemm_nt(_dev(w.A), _dev(w.B), torch.tensor([w.sa], device="cuda"), torch.tensor([w.sb], device="cuda"),
                           a_dtype=fa, b_dtype=fb))
    ref, r, s, _ = oracle.gemm_nt(w.A, w.B, fa, fb, w.sa, w.sb)
    sc = abs(w.sa * w.sb)
    check(d, r, s, sc, ref_bits=ref, what=f"small {M}x{N}x{K}", **random_allowance(w.A, w.B, fa, fb, sc, s))
    rng = np.random.default_rng(M)
    csa = rng.uniform(0.5, 2, M).astype(np.float32)
    csb = rng.uniform(0.5, 2, N).astype(np.float32)
    bias = rng.normal(0, 4, N).astype(np.float32)
    d = gpu_bits(f.gemm_nt_channelwise(_dev(w.A), _dev(w.B), _dev(csa), _dev(csb), _dev(bias), a_dtype=fa, b_dtype=fb))
    ref, r, s = oracle.gemm_nt_channelwise(w.A, w.B, csa, csb, bias, fa, fb)
    _, _, s1, _ = oracle.gemm_nt(w.A, w.B, fa, fb)
    allow = hw_allowance(w.A, w.B, fa, fb, 1.0, s1) * np.outer(csa, csb)
    check(d, r, s, 1.0, ref_bits=ref, what=f"small channelwise {M}x{N}x{K}", allowance=allow,
          max_allowed=random_cap(d.size, K))
    wb = workloads.dense_blockscaled(M, N, K, seed=M + 2 * N + K, lds_pad=5, pad_code=255)
    d = gpu_bits(f.gemm_nt_blockscaled(_dev(wb.A), _dev(wb.B), _dev(wb.sa), _dev(wb.sb), a_dtype=E4M3, b_dtype=E4M3))
    ref, r, s = oracle.gemm_nt_blockscaled(wb.A, wb.B, wb.sa, wb.sb)
    check(d, r, s, 1.0, ref_bits=ref, what=f"small blockscaled {M}x{N}x{K}",
          allowance=hw_allowance_blockscaled(wb.A, wb.B, 0, 0, wb.sa, wb.sb, s), max_allowed=random_cap(d.size, K))

