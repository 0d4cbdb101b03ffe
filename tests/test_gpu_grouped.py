"""GPU parity of the masked and contiguous grouped FP8 GEMMs against the oracle.

Masked form: rows >= m_g of every group must keep their sentinel bytes, and
the NaN-filled activation rows behind them must never reach the result.
Contiguous form: padding rows (grp_idx = -1) must keep their sentinel bytes.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests._parity import check, gpu_bits, random_allowance

pytestmark = pytest.mark.gpu

SENT = 0xDEAD
E4M3, E5M2 = 0, 1


def _lib():
    import fp8_gemm_amd
    return fp8_gemm_amd


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def _sentinel_out(shape):
    t = torch.empty(shape, dtype=torch.int16, device="cuda")
    t.fill_(np.int16(np.uint16(SENT).view(np.int16)))
    return t.view(torch.bfloat16)


def run_masked(w, expected_m=0):
    G, cap, K = w.A.shape
    N = w.B.shape[1]
    print(f"[masked] G={G} cap={cap} N={N} K={K} m={w.masked_m.tolist()[:12]} hint={expected_m}", flush=True)
    f = _lib()
    out = _sentinel_out((G, cap, N))
    f.grouped_gemm_masked(_dev(w.A), _dev(w.B), torch.tensor([w.sa], dtype=torch.float32, device="cuda"),
                          _dev(w.sb), _dev(w.masked_m), out=out, expected_m=expected_m,
                          a_dtype=w.a_fmt, b_dtype=w.b_fmt)
    torch.cuda.synchronize()
    return gpu_bits(out)


def check_masked(w, d, rows_per_group=None, seeded=False):
    """Rows past each count keep the sentinel; valid rows against the oracle
    (random inputs with the capped allowance, seeded configurations on the
    stated bound alone)."""
    G, cap, K = w.A.shape
    m = np.clip(w.masked_m, 0, cap)
    for g in range(G):
        assert (d[g, m[g]:] == SENT).all(), f"group {g}: rows >= m_g were written"
    if rows_per_group is None:
        ref, r, s, _ = oracle.grouped_masked(w.A, w.B, w.masked_m, w.sb, w.a_fmt, w.b_fmt, w.sa)
        for g in range(G):
            if m[g]:
                sc = abs(w.sa * w.sb[g])
                extra = {} if seeded else random_allowance(w.A[g, :m[g]], w.B[g], w.a_fmt, w.b_fmt, sc, s[g, :m[g]])
                check(d[g, :m[g]], r[g, :m[g]], s[g, :m[g]], sc, ref_bits=ref[g, :m[g]], what=f"group {g}", **extra)
        return
    rng = np.random.default_rng(0)
    for g in range(G):
        if not m[g]:
            continue
        rows = np.unique(np.concatenate([[0, m[g] - 1], rng.integers(0, m[g], rows_per_group)]))
        ref, r, s, _ = oracle.gemm_nt(w.A[g, rows], w.B[g], w.a_fmt, w.b_fmt, w.sa, float(w.sb[g]))
        sc = abs(w.sa * w.sb[g])
        extra = {} if seeded else random_allowance(w.A[g, rows], w.B[g], w.a_fmt, w.b_fmt, sc, s)
        check(d[g, rows], r, s, sc, ref_bits=ref, what=f"group {g}", **extra)


COUNTS = [0, 1, 16, 17, 32, 33, 64, 40]


@pytest.mark.parametrize("hint", [0, 16, 32, 64])
def test_masked_all_count_classes(hint):
    """Counts 0 (skipped), 1, a full 16-token block, one past it, 32, 33,
    the capacity, and a hint that is too small (it picks the kernel only)."""
    w = workloads.masked_random(len(COUNTS), 64, 200, 640, seed=41, m_values=COUNTS)
    d = run_masked(w, expected_m=hint)
    check_masked(w, d)


def test_masked_large_counts_take_tiled_kernel():
    w = workloads.masked_random(4, 256, 264, 384, seed=42, m_values=[0, 200, 256, 129])
    assert _lib().plan(1, 256, 264, 384, 4, 0).variant == 2
    d = run_masked(w)
    check_masked(w, d)


@pytest.mark.parametrize("hint", [0, 96, 150])
def test_masked_wide_token_counts(hint):
    """65..192 tokens per group: the swapped kernel with 12 (hints 0 = cap
    192 and 150) or 8 (hint 96) token blocks of 16 in one pass over each
    expert's weights; with 8 blocks the counts above 128 take a second pass.
    Counts on both sides of every pass and block edge, and an empty group."""
    w = workloads.masked_random(9, 192, 264, 640, seed=47, m_values=[0, 65, 96, 128, 129, 160, 192, 1, 17])
    plan = _lib().plan(1, 192, 264, 640, 9, hint)
    assert plan.variant == 3 and plan.token_blocks == (8 if hint == 96 else 12)
    d = run_masked(w, expected_m=hint)
    check_masked(w, d)


@pytest.mark.parametrize("m", [96, 160])
def test_masked_swapab_table_shapes_sampled(m):
    """The swap-AB benchmark table's 16 groups of m = 96 and 160 rows at
    n = 4096, k = 7168 ("One transpose, half the compute", section 4): the
    one-pass swapped kernel, sampled rows of every group under the stated
    bound, every row past the count byte for byte."""
    w = workloads.masked_random(16, 160, 4096, 7168, seed=40, m_values=[m] * 16)
    assert _lib().plan(1, 160, 4096, 7168, 16, m).variant == 3
    d = run_masked(w, expected_m=m)
    check_masked(w, d, rows_per_group=4)


# Seeded random masked configurations (G 1..12, cap 1..300, N a multiple of 8,
# K a multiple of 16, counts U{0..cap}, random hints and formats): the plan is
# the recorded one (variant, token blocks of the swapped kernel: 1..12, and
# the tiled kernel), rows past each count keep the sentinel, and every valid
# row matches the oracle.
@pytest.mark.parametrize("G,cap,N,K,hint,a_fmt,b_fmt,variant,token_blocks", [
    (11, 184, 1128, 928, 18, 0, 1, 3, 2), (6, 162, 1584, 1760, 0, 1, 0, 3, 12), (7, 211, 1344, 256, 0, 0, 1, 2, 0),
    (8, 127, 1408, 96, 0, 0, 0, 3, 8), (8, 39, 32, 480, 0, 0, 1, 3, 4), (11, 15, 2432, 160, 0, 1, 1, 3, 1),
    (12, 69, 2128, 544, 54, 1, 0, 3, 4), (1, 219, 2408, 1856, 0, 0, 0, 2, 0), (7, 142, 1208, 2336, 0, 0, 0, 3, 12),
    (7, 30, 304, 1152, 0, 1, 0, 3, 2),
])
def test_masked_random_configs(G, cap, N, K, hint, a_fmt, b_fmt, variant, token_blocks):
    p = _lib().plan(1, cap, N, K, G, hint)
    assert (p.variant, p.token_blocks) == (variant, token_blocks)
    w = workloads.masked_random(G, cap, N, K, seed=G * cap + N + K, a_fmt=a_fmt, b_fmt=b_fmt)
    d = run_masked(w, expected_m=hint)
    check_masked(w, d)


def test_masked_clamps_counts():
    w = workloads.masked_random(3, 32, 128, 256, seed=43, m_values=[-5, 1000, 7])
    d = run_masked(w)
    check_masked(w, d)


def test_masked_all_groups_empty():
    w = workloads.masked_random(5, 64, 128, 256, seed=44, m_values=[0] * 5)
    d = run_masked(w)
    assert (d == SENT).all()


@pytest.mark.parametrize("a_fmt,b_fmt", [(E4M3, E5M2), (E5M2, E5M2)])
def test_masked_formats(a_fmt, b_fmt):
    w = workloads.masked_random(3, 64, 136, 512, seed=45, m_values=[5, 31, 64], a_fmt=a_fmt, b_fmt=b_fmt)
    d = run_masked(w)
    check_masked(w, d)


def test_masked_decode_config_sampled():
    """G=32, cap=64, N=4096, K=7168, m_g ~ U{0..32}: every untouched row is
    checked byte for byte, valid rows are sampled per group."""
    w = workloads.masked_decode()
    d = run_masked(w, expected_m=32)
    check_masked(w, d, rows_per_group=3, seeded=True)


def test_grouped_equals_per_group_dense():
    w = workloads.masked_random(3, 64, 256, 1024, seed=46, m_values=[64, 20, 3])
    d = run_masked(w)
    f = _lib()
    for g in range(3):
        m = int(w.masked_m[g])
        out = f.gemm_nt(_dev(w.A[g, :m]), _dev(w.B[g]), torch.tensor([w.sa], dtype=torch.float32, device="cuda"),
                        torch.tensor([w.sb[g]], dtype=torch.float32, device="cuda"), a_dtype=E4M3, b_dtype=E4M3)
        torch.cuda.synchronize()
        dd = gpu_bits(out)
        ref, r, s, _ = oracle.gemm_nt(w.A[g, :m], w.B[g], sa=w.sa, sb=float(w.sb[g]))
        sc = abs(w.sa * w.sb[g])
        extra = random_allowance(w.A[g, :m], w.B[g], E4M3, E4M3, sc, s)
        check(dd, r, s, sc, ref_bits=ref, what=f"dense group {g}", **extra)
        check(d[g, :m], r, s, sc, ref_bits=ref, what=f"grouped group {g}", **extra)


# ---------------------------------------------------------------------------
# Contiguous grouped
# ---------------------------------------------------------------------------

def run_contig(w):
    M_total, K = w.A.shape
    G, N, _ = w.B.shape
    print(f"[contig] M_total={M_total} G={G} N={N} K={K}", flush=True)
    f = _lib()
    out = _sentinel_out((M_total, N))
    f.grouped_gemm_contig(_dev(w.A), _dev(w.B), torch.tensor([w.sa], dtype=torch.float32, device="cuda"),
                          _dev(w.sb), _dev(w.grp_idx), out=out, a_dtype=w.a_fmt, b_dtype=w.b_fmt)
    torch.cuda.synchronize()
    return gpu_bits(out)


def check_contig(w, d, sample_rows=None, seeded=False):
    pad = w.grp_idx < 0
    assert (d[pad] == SENT).all(), "padding rows were written"
    if sample_rows is None:
        ref, r, s, _ = oracle.grouped_contig(w.A, w.B, w.grp_idx, w.sb, w.a_fmt, w.b_fmt, w.sa)
        for g in np.unique(w.grp_idx[~pad]):
            rg = np.flatnonzero(w.grp_idx == g)
            sc = abs(w.sa * w.sb[g])
            extra = {} if seeded else random_allowance(w.A[rg], w.B[g], w.a_fmt, w.b_fmt, sc, s[rg])
            check(d[rg], r[rg], s[rg], sc, ref_bits=ref[rg], what=f"contig expert {g}", **extra)
        return
    rng = np.random.default_rng(1)
    real_rows = np.flatnonzero(~pad)
    rows = np.unique(rng.choice(real_rows, size=min(sample_rows, real_rows.size), replace=False))
    for g in np.unique(w.grp_idx[rows]):
        rg = rows[w.grp_idx[rows] == g]
        ref, r, s, _ = oracle.gemm_nt(w.A[rg], w.B[g], w.a_fmt, w.b_fmt, w.sa, float(w.sb[g]))
        sc = abs(w.sa * w.sb[g])
        extra = {} if seeded else random_allowance(w.A[rg], w.B[g], w.a_fmt, w.b_fmt, sc, s)
        check(d[rg], r, s, sc, ref_bits=ref, what=f"contig expert {g}", **extra)


def test_contig_small():
    w = workloads.contig_random(tokens=300, topk=2, G=5, N=264, K=512, seed=51)
    d = run_contig(w)
    check_contig(w, d)


def test_contig_empty_experts_and_tail():
    w = workloads.contig_random(tokens=0, topk=1, G=4, N=128, K=256, seed=52, counts=[0, 129, 0, 1])
    assert w.A.shape[0] == 256 + 128
    d = run_contig(w)
    check_contig(w, d)


def test_contig_expert_changes_at_odd_and_even_blocks():
    """Runs of 128 | 256 | 128 | 128 | 384 | 128 rows (one empty expert): the
    expert changes both inside 256-row tiles (at odd 128-row blocks) and
    between them; ragged N and K."""
    w = workloads.contig_random(tokens=0, topk=1, G=7, N=264, K=400, seed=54, counts=[128, 256, 1, 127, 0, 300, 5])
    assert w.A.shape[0] == 9 * 128
    d = run_contig(w)
    check_contig(w, d)


def test_contig_all_padding_halves():
    """A 256-row tile whose first, or second, 128-row half is all padding."""
    w = workloads.contig_random(tokens=0, topk=1, G=4, N=256, K=256, seed=55, counts=[100, 256, 300, 128])
    assert w.A.shape[0] == 7 * 128
    w.grp_idx[0:128] = -1          # first half of tile 0 all padding; expert 1 fills its second half
    w.grp_idx[640:768] = -1        # second half of tile 2 all padding
    d = run_contig(w)
    check_contig(w, d)


def test_contig_long_runs():
    """Run-aligned tiles: a run of 70 128-row blocks starting at an odd block
    (its tiles start at odd blocks, and finding a tile start scans back over
    more than 64 blocks), then a 3-block run (a 256-row tile and a 128-row
    one) and a single-block run; N tail inside a 256-column tile."""
    w = workloads.contig_random(tokens=0, topk=1, G=4, N=136, K=256, seed=56, counts=[100, 70 * 128 - 5, 300, 1])
    assert w.A.shape[0] == (1 + 70 + 3 + 1) * 128
    d = run_contig(w)
    check_contig(w, d)


def test_contig_formats():
    w = workloads.contig_random(tokens=200, topk=1, G=3, N=136, K=384, seed=53, a_fmt=E5M2, b_fmt=E4M3)
    d = run_contig(w)
    check_contig(w, d)


# Seeded random contiguous configurations (1..16 experts, Dirichlet-multinomial
# counts with empty experts, N a multiple of 8, K a multiple of 16, random
# formats): padding rows keep the sentinel and every routed row matches the
# oracle.
@pytest.mark.parametrize("tokens,topk,G,N,K,a_fmt,b_fmt", [
    (429, 3, 13, 104, 208, 1, 1), (920, 3, 8, 640, 880, 1, 0), (111, 4, 4, 112, 400, 0, 0),
    (1035, 4, 10, 224, 1152, 1, 0), (366, 3, 7, 3856, 96, 1, 0), (1081, 3, 1, 1240, 272, 0, 0),
    (903, 2, 1, 224, 160, 1, 0), (308, 1, 16, 3904, 192, 1, 0),
])
def test_contig_random_configs(tokens, topk, G, N, K, a_fmt, b_fmt):
    w = workloads.contig_random(tokens, topk, G, N, K, seed=tokens + G + N + K, a_fmt=a_fmt, b_fmt=b_fmt)
    d = run_contig(w)
    check_contig(w, d)


def test_contig_prefill_config_sampled():
    """8192 tokens x top-8 over 32 experts, N=4096, K=7168."""
    w = workloads.contig_prefill()
    d = run_contig(w)
    check_contig(w, d, sample_rows=192, seeded=True)
