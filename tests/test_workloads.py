"""Seeded input generators: determinism and stated distributions (CPU only)."""
import hashlib

import numpy as np

import workloads


def _h(a):
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def test_dense_generator_is_deterministic():
    a = workloads.dense_random(64, 48, 256, seed=3)
    b = workloads.dense_random(64, 48, 256, seed=3)
    assert _h(a.A) == _h(b.A) and _h(a.B) == _h(b.B)
    c = workloads.dense_random(64, 48, 256, seed=4)
    assert _h(a.A) != _h(c.A)


def test_quantize_saturates_and_rounds():
    x = np.array([1000.0, -1000.0, 1.0, 1.0625, 1.1875, 0.0], np.float32)
    q = workloads.quantize(x, workloads.E4M3)
    assert list(q) == [0x7E, 0xFE, 0x38, 0x38, 0x3A, 0x00]   # 1.0625 ties to 1.0; 1.1875 ties to 1.25
    q2 = workloads.quantize(np.array([1e9, -1e9], np.float32), workloads.E5M2)
    assert list(q2) == [0x7B, 0xFB]


def test_masked_generator_layout():
    w = workloads.masked_random(5, 8, 16, 64, seed=2, m_max=6)
    assert w.A.shape == (5, 8, 64) and w.B.shape == (5, 16, 64)
    for g in range(5):
        m = int(w.masked_m[g])
        assert 0 <= m <= 6
        assert (w.A[g, m:] == 0x7F).all()
        assert not (w.A[g, :m] == 0x7F).any()
    # weights are amax-scaled: the largest magnitude code of each expert is 448
    assert all(int((w.B[g] & 0x7F).max()) == 0x7E for g in range(5))


def test_contig_generator_layout():
    w = workloads.contig_random(tokens=100, topk=4, G=6, N=8, K=32, seed=5, align=16)
    assert int(w.counts.sum()) == 400
    assert w.A.shape[0] % 16 == 0
    real = w.grp_idx >= 0
    assert int(real.sum()) == 400
    assert (w.A[~real] == 0x7F).all()
    # groups are contiguous, in order, each starting on an aligned row
    starts = [int(np.argmax(w.grp_idx == g)) for g in range(6) if w.counts[g] > 0]
    assert all(s % 16 == 0 for s in starts) and starts == sorted(starts)
    # every aligned block holds one expert only (or padding)
    for b in range(0, w.A.shape[0], 16):
        ids = set(int(v) for v in w.grp_idx[b:b + 16]) - {-1}
        assert len(ids) <= 1
