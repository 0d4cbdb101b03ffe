"""GPU parity of the block-scaled masked grouped GEMM
(fp8_grouped_gemm_masked_blockscaled) against the CPU oracle, through the C ABI:
the swapped streaming kernel (hint <= 64) and the tiled kernel (larger hints).
Rows past each expert's count hold NaN codes and NaN scales, as does every
scale array's padding; they must never reach a written output, and rows past
the count must keep the sentinel."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests._parity import check, gpu_bits, hw_allowance_blockscaled, random_cap

pytestmark = pytest.mark.gpu

SENT = 0xDEAD


def _f():
    import fp8_gemm_amd
    return fp8_gemm_amd


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def run(w, hint):
    G, cap, K = w.A.shape
    N = w.B.shape[1]
    print(f"[masked bs] G={G} cap={cap} N={N} K={K} hint={hint} m={list(w.masked_m)[:8]}", flush=True)
    out = torch.full((G, cap, N), 0, dtype=torch.int16, device="cuda")
    out.fill_(SENT - 65536)
    out = out.view(torch.bfloat16)
    _f().grouped_gemm_masked_blockscaled(_dev(w.A), _dev(w.B), _dev(w.sa), _dev(w.sb), _dev(w.masked_m), out=out,
                                         expected_m=hint, a_dtype=0, b_dtype=0)
    torch.cuda.synchronize()
    return gpu_bits(out)


def check_groups(w, d, rows=None):
    """Random inputs: the capped truncation allowance."""
    G, cap, K = w.A.shape
    for g in range(G):
        m = int(min(max(w.masked_m[g], 0), cap))
        assert (d[g, m:] == SENT).all(), f"group {g}: a row past the count was written"
        if not m:
            continue
        ref, r, s = oracle.gemm_nt_blockscaled(w.A[g, :m], w.B[g], w.sa[g], w.sb[g])
        check(d[g, :m], r, s, 1.0, ref_bits=ref, what=f"{w.name} group {g}",
              allowance=hw_allowance_blockscaled(w.A[g, :m], w.B[g], 0, 0, w.sa[g], w.sb[g], s),
              max_allowed=random_cap(s.size, K))


@pytest.mark.parametrize("hint", [0, 16, 32, 64])
def test_swap_counts(hint):
    w = workloads.masked_blockscaled(8, 64, 520, 400, seed=60 + hint, m_values=[0, 1, 16, 17, 32, 33, 64, 40],
                                     lds_pad=5)
    check_groups(w, run(w, hint))


@pytest.mark.parametrize("hint", [96, 0])
def test_wide_token_counts(hint):
    """65..192 tokens per group with block scales: the swapped kernel with 8
    (hint 96; counts above 128 take a second pass) or 12 (hint 0 = cap 192)
    token blocks; NaN codes and scales behind every count."""
    w = workloads.masked_blockscaled(6, 192, 520, 400, seed=66 + hint, m_values=[0, 65, 128, 129, 192, 100],
                                     lds_pad=5)
    p = _f().plan(1, 192, 520, 400, 6, hint)
    assert p.variant == 3 and p.token_blocks == (8 if hint == 96 else 12)
    check_groups(w, run(w, hint))


def test_tiled_large_counts():
    w = workloads.masked_blockscaled(3, 256, 264, 272, seed=64, m_values=[256, 129, 0], lds_pad=3)
    assert _f().plan(1, 256, 264, 272, 3, 200).variant == 2
    check_groups(w, run(w, 200))


def test_scale_shift_is_bit_exact():
    """Doubling one token row's K block in one expert (and decrementing its
    scale), or one 128-row weight block of an expert, leaves D unchanged."""
    rng = np.random.default_rng(65)
    G, cap, N, K = 3, 32, 264, 384
    w = workloads.masked_blockscaled(G, cap, N, K, seed=65, m_values=[32, 20, 5])
    e = rng.integers(1, 12, size=w.A.shape)
    w.A[:] = ((rng.integers(0, 2, size=w.A.shape) << 7) | (e << 3) | rng.integers(0, 8, size=w.A.shape)).astype(np.uint8)
    e = rng.integers(1, 12, size=w.B.shape)
    w.B[:] = ((rng.integers(0, 2, size=w.B.shape) << 7) | (e << 3) | rng.integers(0, 8, size=w.B.shape)).astype(np.uint8)
    w.sa[w.sa != 255] = 120
    w.sb[w.sb != 255] = 118
    base = run(w, 32)
    A2, sa2 = w.A.copy(), w.sa.copy()
    A2[1, 7, 128:256] += 8
    sa2[1, 1, 7] -= 1
    w2 = workloads.MaskedBlockScaled(A2, w.B, sa2, w.sb, w.masked_m, name="shift A")
    assert np.array_equal(run(w2, 32), base)
    B2, sb2 = w.B.copy(), w.sb.copy()
    B2[2, 128:256, 256:384] += 8
    sb2[2, 1, 2] -= 1
    w3 = workloads.MaskedBlockScaled(w.A, B2, w.sa, sb2, w.masked_m, name="shift B")
    assert np.array_equal(run(w3, 32), base)


def test_decode_config_sampled():
    """G=32, cap=64, N=4096, K=7168, m_g ~ U{0..32}: every row past a count keeps
    the sentinel; sampled valid rows meet the stated bound."""
    w = workloads.masked_decode_blockscaled()
    d = run(w, 32)
    rng = np.random.default_rng(9)
    for g in range(32):
        m = int(w.masked_m[g])
        assert (d[g, m:] == SENT).all()
        if not m:
            continue
        rows = np.unique(rng.integers(0, m, 2))
        cols = rng.integers(0, 4096, 256)
        ii = np.repeat(rows, cols.size)
        jj = np.tile(cols, rows.size)
        ref, r, s = oracle.gemm_nt_blockscaled_points(w.A[g], w.B[g], w.sa[g], w.sb[g], ii, jj)
        check(d[g][ii, jj], r, s, 1.0, ref_bits=ref, what=f"decode bs group {g}")


def run_contig(w):
    M, K = w.A.shape
    G, N, _ = w.B.shape
    print(f"[contig bs] M_total={M} G={G} N={N} K={K}", flush=True)
    out = torch.full((M, N), SENT - 65536, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    _f().grouped_gemm_contig_blockscaled(_dev(w.A), _dev(w.B), _dev(w.sa), _dev(w.sb), _dev(w.grp_idx), out=out,
                                         a_dtype=0, b_dtype=0)
    torch.cuda.synchronize()
    return gpu_bits(out)


def check_contig(w, d, rows=None, seeded=False):
    pad = w.grp_idx < 0
    assert (d[pad] == SENT).all(), "a padding row was written"
    real = np.flatnonzero(~pad)
    if rows is not None:
        real = np.unique(np.random.default_rng(3).choice(real, size=min(rows, real.size), replace=False))
    for g in np.unique(w.grp_idx[real]):
        rg = real[w.grp_idx[real] == g]
        ref, r, s = oracle.gemm_nt_blockscaled(w.A[rg], w.B[g], w.sa[:, rg], w.sb[g])
        extra = {} if seeded else {
            "allowance": hw_allowance_blockscaled(w.A[rg], w.B[g], 0, 0, w.sa[:, rg], w.sb[g], s),
            "max_allowed": random_cap(s.size, w.A.shape[1])}
        check(d[rg], r, s, 1.0, ref_bits=ref, what=f"{w.name} expert {g}", **extra)


@pytest.mark.parametrize("counts", [[128, 256, 1, 127, 0, 300, 5], [100, 256, 300, 128]])
def test_contig_expert_changes(counts):
    """Expert changes inside 256-row tiles (the second-block workgroups) and
    between them, ragged N and K, NaN padding rows and scales."""
    w = workloads.contig_blockscaled(0, 1, len(counts), 264, 400, seed=70 + len(counts), counts=counts, lds_pad=6)
    check_contig(w, run_contig(w))


def _random_counts(seed, G, long_run):
    """Per-expert counts: empty experts, partial blocks, runs of a few blocks
    and, with long_run, one run of more than 64 blocks (the slot's backward
    scan then takes further rounds)."""
    rng = np.random.default_rng(seed)
    c = rng.choice([0, 1, 127, 128, 129, 255, 256, 257, 384, 500, 1000], size=G).astype(np.int64)
    c += rng.integers(0, 40, size=G) * (c > 0)
    if long_run:
        c[int(rng.integers(0, G))] = 66 * 128 + int(rng.integers(1, 128))
    return c


# Seeded random run layouts for the run-aligned tiles: the expert changes at
# odd and even 128-row blocks, runs of 1 to 67 blocks, empty experts; N a
# multiple of 8 with a tail inside a 256-column tile, K a multiple of 16.
@pytest.mark.parametrize("seed,G,N,K,long_run", [
    (101, 9, 264, 400, False), (102, 12, 136, 256, False), (103, 5, 520, 144, True),
    (104, 7, 392, 1040, False), (105, 3, 1032, 128, True), (106, 11, 24, 272, False),
])
def test_contig_random_runs(seed, G, N, K, long_run):
    counts = _random_counts(seed, G, long_run)
    w = workloads.contig_blockscaled(0, 1, G, N, K, seed=seed, counts=counts.tolist(), lds_pad=seed % 9)
    print(f"[contig bs random] counts={counts.tolist()}", flush=True)
    check_contig(w, run_contig(w))


def test_contig_prefill_sampled():
    w = workloads.contig_blockscaled(8192, 8, 32, 4096, 7168, seed=9)
    check_contig(w, run_contig(w), rows=256, seeded=True)
