"""Pins of this build's work formulas and workload shapes to numbers the pages print
(tests/golden/pages_numbers.txt, each line cited there).  CPU only."""
import os

import numpy as np

import workloads

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "pages_numbers.txt")


def _lines(tag):
    out = []
    for line in open(GOLDEN):
        line = line.split("#")[0].strip()
        if line.startswith(tag + " "):
            out.append(line.split()[1:])
    return out


def test_intensity_example():
    """2 n^3 FLOPs over 3 n^2 bytes: the printed n = 1024 example and the printed
    Hopper compute-to-bandwidth ratio, to their printed rounding."""
    (ex, hopper) = _lines("intensity")
    n = int(ex[0].split("=")[1])
    printed = float(ex[1].split("~")[1])
    assert abs((2 * n ** 3) / (3 * n ** 2) - printed) / printed < 0.01
    tf = float(hopper[0].split("=")[1])
    tbs = float(hopper[1].split("=")[1])
    printed = float(hopper[2].split("~")[1])
    assert abs(tf / tbs - printed) / printed < 0.01


def test_bench_work_formulas_match_the_pages():
    """bench.py counts 2 M N K FLOPs for a dense GEMM (the pages' 2 n^3) and one pass
    over A, B and D (the pages' 3 n^2 bytes with 1-byte elements; D here is BF16, 2
    bytes an element, so 4 n^2)."""
    import bench
    n = 4096
    flops, nbytes = bench.dense_work(n, n, n)
    assert flops == 2 * n ** 3
    assert nbytes == 4 * n ** 2
    f2, b2 = bench.dense_work(3, 5, 7)
    assert f2 == 2 * 3 * 5 * 7 and b2 == 3 * 7 + 5 * 7 + 2 * 3 * 5


def test_swapab_table_gains_and_the_masked_workload_shape():
    """The printed gains are swapped / original - 1 of the printed rates, and the masked
    decode workload uses the table's first shape (n = 4096, k = 7168, m up to 32)."""
    rows = _lines("swapab")
    assert len(rows) == 6
    for m, n, k, orig, swp, gain in rows:
        assert abs((float(swp) / float(orig) - 1) * 100 - float(gain)) < 0.1, (m, n, k)
    m, n, k = (int(v) for v in rows[0][:3])
    w = workloads.masked_decode()
    assert w.B.shape[1:] == (n, k)
    assert int(np.clip(w.masked_m, 0, None).max()) <= m
