"""Seeded random sweep of every FP8 entry point against the oracle.

Each case draws its own configuration from a generator seeded with its index:
dense (few-token and tiled shapes), block-scaled dense, per-channel dense,
masked grouped, contiguous grouped, the block-scaled masked and contiguous
forms, the BF16 comparison path, and the allocation-free dense entry point on
few-token shapes (with and without split K); shapes, counts, formats, scale-array padding and expected-count hints
at random, within each entry point's layout rules.  Every output goes through
the same checks as the targeted tests: the stated bound, with the capped
matrix-core truncation allowance for random data, and sentinels on every row
the call must not write.  (Random shapes of this kind, in the block-scaled
dense tests, exposed a race between a ring slot's reads and its refill in the
few-token kernel.)
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests._parity import check, random_allowance
from tests import test_gpu_bf16 as TBF
from tests import test_gpu_blockscaled as TB
from tests import test_gpu_channelwise as TC
from tests import test_gpu_dense as TD
from tests import test_gpu_grouped as TG
from tests import test_gpu_grouped_blockscaled as TGB

pytestmark = pytest.mark.gpu

KINDS = ("dense", "blockscaled", "channelwise", "masked", "contig", "masked_bs", "contig_bs", "bf16", "noalloc")
CASES = 10                                          # per entry point


def _draw(rng, limit, make):
    while True:
        cfg = make()
        if cfg[-1] <= limit:
            return cfg[:-1]


@pytest.mark.parametrize("i", range(len(KINDS) * CASES))
def test_random_entry_point(i):
    kind = KINDS[i % len(KINDS)]
    rng = np.random.default_rng(9000 + i)
    ri = lambda a, b: int(rng.integers(a, b))
    fa, fb = ri(0, 2), ri(0, 2)
    rows = lambda: ri(1, 65) if rng.random() < 0.4 else ri(65, 3000)
    if kind == "dense":
        M, N, K = _draw(rng, 3e9, lambda: (m := rows(), n := ri(1, 9000), k := 16 * ri(1, 160), m * n * k))
        print(f"[sweep {i}] dense M={M} N={N} K={K} fmt=({fa},{fb})", flush=True)
        TD._check_dense(workloads.dense_random(M, N, K, seed=i, a_fmt=fa, b_fmt=fb, scales=(0.75, 1.5)),
                        f"sweep {i}")
    elif kind == "blockscaled":
        M, N, K = _draw(rng, 3e9, lambda: (m := rows(), n := 8 * ri(1, 1100), k := 16 * ri(1, 160), m * n * k))
        w = workloads.dense_blockscaled(M, N, K, seed=i, a_fmt=fa, b_fmt=fb, lds_pad=ri(0, 9))
        TB.check_full(w, TB.run_bs(w))
    elif kind == "channelwise":
        M, N, K = _draw(rng, 2e9, lambda: (m := rows(), n := ri(1, 9000), k := 16 * ri(1, 120), m * n * k))
        which = "".join(c for c in "abc" if rng.random() < 0.6) or "c"
        TC.test_channelwise_matches_oracle(M, N, K, fa, fb, which)
    elif kind == "noalloc":
        M, N, K = ri(1, 65), 8 * ri(1, 2000), 16 * ri(16, 600)
        print(f"[sweep {i}] no-alloc M={M} N={N} K={K} fmt=({fa},{fb}) k_splits={TD._lib().plan(0, M, N, K).k_splits}",
              flush=True)
        w = workloads.dense_random(M, N, K, seed=i, a_fmt=fa, b_fmt=fb, scales=(0.75, 1.5))
        out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        TD._lib().gemm_nt(TD._dev(w.A), TD._dev(w.B), TD._scale(w.sa), TD._scale(w.sb), out=out,
                          a_dtype=fa, b_dtype=fb, no_alloc=True)
        torch.cuda.synchronize()
        d = TD.gpu_bits(out)
        ref, r, s, _ = oracle.gemm_nt(w.A, w.B, fa, fb, w.sa, w.sb)
        sc = abs(w.sa * w.sb)
        check(d, r, s, sc, ref_bits=ref, what=f"sweep {i} no-alloc", **random_allowance(w.A, w.B, fa, fb, sc, s))
    elif kind == "bf16":
        M, N, K = _draw(rng, 1.5e9, lambda: (m := rows(), n := ri(1, 6000), k := 8 * ri(1, 200), m * n * k))
        w = workloads.dense_bf16_random(M, N, K, seed=i)
        TBF._check_bf16(w.A, w.B, f"sweep {i} bf16 {M}x{N}x{K}")
    elif kind in ("masked", "masked_bs"):
        G, cap, N, K = _draw(rng, 3e9, lambda: (g := ri(1, 17), c := ri(1, 300), n := 8 * ri(1, 500),
                                                 k := 16 * ri(1, 160), g * c * n * k))
        hint = int(rng.choice([0, ri(1, cap + 1)]))
        if kind == "masked":
            w = workloads.masked_random(G, cap, N, K, seed=i, a_fmt=fa, b_fmt=fb)
            TG.check_masked(w, TG.run_masked(w, expected_m=hint))
        else:
            w = workloads.masked_blockscaled(G, cap, N, K, seed=i, lds_pad=ri(0, 9))
            TGB.check_groups(w, TGB.run(w, hint))
    else:
        G, tokens, topk, N, K = _draw(rng, 3e9, lambda: (g := ri(1, 20), t := ri(0, 1500), tk := ri(1, 5),
                                                          n := 8 * ri(1, 500), k := 16 * ri(1, 160),
                                                          (t * tk + 128 * g) * n * k))
        if kind == "contig":
            w = workloads.contig_random(tokens, topk, G, N, K, seed=i, a_fmt=fa, b_fmt=fb)
            TG.check_contig(w, TG.run_contig(w))
        else:
            w = workloads.contig_blockscaled(tokens, topk, G, N, K, seed=i, lds_pad=ri(0, 9))
            TGB.check_contig(w, TGB.run_contig(w))
