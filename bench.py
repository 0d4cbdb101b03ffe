"""Benchmark of the FP8 GEMM path on one MI355X.

Metric: FP8 TFLOP/s (and fraction of the MFMA FP8 peak) of the dense 4096^3
E4M3 GEMM; HBM GB/s of the masked grouped decode GEMM (m_g <= 32).

One step = one dense 4096^3 GEMM (D = bf16(sa*sb*A.B^T), inputs resident in
HBM).  `value` is the whole-job rate over the timed steps.  The same run also
times, each in its own timed loop: the masked grouped decode GEMM (G=32,
cap=64, N=4096, K=7168, m_g ~ U{0..32}) against the HBM roofline, the
contiguous grouped prefill GEMM, the 256^3 GEMM (latency), the E5M2 4096^3
GEMM, the block-scaled and the per-channel 4096^3 GEMMs, the dense few-token
(decode) GEMMs against the HBM roofline and the eight transformer-projection
shapes.

Timing ("the median of repeated event-timed launches"): each leg's average
launch duration is the interval between two HIP events recorded around its K
back-to-back launches on the stream the kernels run on (torch's current
stream, which the library is handed), divided by K.  Each leg then runs 30
further windows of L back-to-back launches (L chosen so a window lasts at
least 0.5 ms), with an event between windows; the first 5 windows are
discarded and the median, p10 and p90 of the per-launch time over the other
25 are reported.

CPU baseline: the oracle, timed after the GPU legs on the host threads this
process may use (its CPU affinity, capped by OMP_NUM_THREADS where that is
set), on a bounded sample of each configuration (rows of the problem, whole
problems where they are small), about 20-30 s in all.

Counters: `--profile-run` launches each profiled workload a few times eagerly
(no timing) for rocprofv3; `--counters-summary` turns one kernel-trace pass and
three --pmc passes (FETCH_SIZE; WRITE_SIZE; SQ/GRBM counters) into
profiles/<kernel>_<workload>_counters.txt, the HBM byte counters scaled by what
they read for a 1 GiB copy of known size.

    python bench.py [--gpus 1] [--steps 200] [--warmup 20] [--only NAME ...] [--no-cpu]
    python bench.py --profile-run [--profile-targets NAME ...]
    python bench.py --counters-summary TRACE_DIR FETCH_DIR WRITE_DIR SQ_DIR --counters-command "..."
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP8_TFLOPS = 5000.0      # MI355X dense FP8 matrix peak (no sparsity)
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense BF16 matrix peak (no sparsity)
SIMDS = 1024                  # 256 CUs x 4 SIMDs
METRIC = "FP8 TFLOPS (+% MFMA peak) dense 4096³; HBM GB/s masked grouped m≤32"
PROFILE_DIR = os.path.join(ROOT, "profiles")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("kernels.hpp", "device_common.hpp", "fp8_gemm.hip"):
        with open(os.path.join(ROOT, "fp8_gemm_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_counters(name: str):
    """Per-launch figures recorded from rocprofv3 for counter target `name`, or
    None when no summary exists or the kernels changed since it was taken."""
    path = os.path.join(PROFILE_DIR, f"{COUNTER_TARGETS[name][0]}_counters.txt")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"kernel_source_hash:\s*(\w+)", text)
    if not m_hash or m_hash.group(1) != kernel_source_hash():
        return None
    out = {}
    for key in ("hbm_bytes_per_launch", "mfma_busy_fraction", "effective_clock_ghz", "lds_bank_conflict_fraction"):
        m = re.search(rf"{key}:\s*([0-9.eE+-]+)", text)
        if m:
            out[key] = float(m.group(1))
    return out


def _stats(vals):
    import numpy as np

    v = np.asarray(vals, dtype=np.float64)
    return {"median_ms": float(np.median(v)), "p10_ms": float(np.percentile(v, 10)),
            "p90_ms": float(np.percentile(v, 90))}


class Timer:
    """Times `fn` (which launches work on torch's current stream): at least
    `warmup` untimed calls and at least `min_warm_s` seconds of them (the GPU
    clock ramps up over the first few milliseconds of load after idle), then
    exactly `steps` back-to-back calls between one pair of HIP events recorded
    on that stream, with a synchronize on both sides of the timed region.  The
    average launch duration is the event interval over `steps`.  Then the
    spread: WINDOWS windows of back-to-back calls, an event between windows,
    the first DISCARD dropped."""

    WINDOWS, DISCARD, MIN_WINDOW_MS = 30, 5, 0.5

    def __init__(self, torch, min_warm_s=0.25):
        self.torch = torch
        self.min_warm_s = min_warm_s

    def run(self, fn, steps, warmup):
        torch = self.torch
        t0 = time.perf_counter()
        done = 0
        while done < warmup or time.perf_counter() - t0 < self.min_warm_s:
            fn()
            done += 1
            if done % 16 == 0:
                torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        mean = e0.elapsed_time(e1) / steps
        out = {"wall_s": wall, "kernel_ms_mean": mean, "warmup_calls": done}
        out.update(self.spread(fn, mean))
        return out

    def spread(self, fn, mean_ms):
        torch = self.torch
        per = max(2, int(math.ceil(self.MIN_WINDOW_MS / max(mean_ms, 1e-4))))
        stream = torch.cuda.current_stream()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(self.WINDOWS + 1)]
        torch.cuda.synchronize()
        ev[0].record(stream)
        for w in range(self.WINDOWS):
            for _ in range(per):
                fn()
            ev[w + 1].record(stream)
        torch.cuda.synchronize()
        vals = [ev[w].elapsed_time(ev[w + 1]) / per for w in range(self.DISCARD, self.WINDOWS)]
        out = _stats(vals)
        out.update({"windows": self.WINDOWS - self.DISCARD, "launches_per_window": per})
        return out

    def run_graph(self, fn, n, replays=None):
        """For launches shorter than the host's per-call cost (~10 us through
        Python): fn(j) for j < n captured once in a graph, which is replayed
        for at least `min_warm_s` seconds, then WINDOWS times with an event
        between replays on the replay stream.  The average launch duration is
        the interval over the last WINDOWS - DISCARD replays over their
        launches; median, p10 and p90 are per replay."""
        torch = self.torch
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for j in range(3):
                fn(j)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for j in range(n):
                fn(j)
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < self.min_warm_s:
            g.replay()
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(self.WINDOWS + 1)]
        ev[0].record(stream)
        for w in range(self.WINDOWS):
            g.replay()
            ev[w + 1].record(stream)
        torch.cuda.synchronize()
        del g
        vals = [ev[w].elapsed_time(ev[w + 1]) / n for w in range(self.DISCARD, self.WINDOWS)]
        out = _stats(vals)
        kept = self.WINDOWS - self.DISCARD
        out.update({"kernel_ms_mean": ev[self.DISCARD].elapsed_time(ev[self.WINDOWS]) / (kept * n),
                    "launches": kept * n, "windows": kept, "launches_per_window": n})
        return out


def timing_fields(t, scale=1.0):
    """The spread of a Timer result in microseconds (times scale)."""
    return {"us_median": t["median_ms"] * 1e3 * scale, "us_p10": t["p10_ms"] * 1e3 * scale,
            "us_p90": t["p90_ms"] * 1e3 * scale, "windows": t["windows"],
            "launches_per_window": t["launches_per_window"]}
def dev(torch, x):
    return torch.from_numpy(x).cuda()


def dense_work(M, N, K):
    """Algorithmic work of one dense GEMM: 2 M N K FLOPs, and one pass over the
    FP8 operands (1 byte an element) and the BF16 output (2 bytes)."""
    return 2.0 * M * N * K, float(M * K + N * K + 2 * M * N)


def bench_dense(torch, f, w, steps, warmup, timer):
    a, b = dev(torch, w.A), dev(torch, w.B)
    sa = torch.tensor([w.sa], dtype=torch.float32, device="cuda")
    sb = torch.tensor([w.sb], dtype=torch.float32, device="cuda")
    M, N, K = w.shape
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    fn = lambda: f.gemm_nt(a, b, sa, sb, out=out, a_dtype=w.a_fmt, b_dtype=w.b_fmt)
    t = timer.run(fn, steps, warmup)
    flops, nbytes = dense_work(M, N, K)
    t["flops"] = flops
    t["tflops_wall"] = flops * steps / t["wall_s"] / 1e12
    t["tflops_kernel"] = flops / (t["kernel_ms_mean"] * 1e-3) / 1e12
    t["bytes"] = nbytes
    del a, b, out
    return t


def bench_blockscaled(torch, f, w, steps, warmup, timer):
    a, b = dev(torch, w.A), dev(torch, w.B)
    sa, sb = dev(torch, w.sa), dev(torch, w.sb)
    M, N, K = w.shape
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    fn = lambda: f.gemm_nt_blockscaled(a, b, sa, sb, out=out, a_dtype=w.a_fmt, b_dtype=w.b_fmt)
    t = timer.run(fn, steps, warmup)
    flops = 2.0 * M * N * K
    t["flops"] = flops
    t["tflops_kernel"] = flops / (t["kernel_ms_mean"] * 1e-3) / 1e12
    del a, b, sa, sb, out
    return t


def bench_channelwise(torch, f, w, steps, warmup, timer):
    import numpy as np

    M, N, K = w.shape
    rng = np.random.default_rng(12)
    a, b = dev(torch, w.A), dev(torch, w.B)
    sa = dev(torch, rng.uniform(0.5, 2, M).astype(np.float32))
    sb = dev(torch, rng.uniform(0.5, 2, N).astype(np.float32))
    bias = dev(torch, rng.normal(0, 1, N).astype(np.float32))
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    fn = lambda: f.gemm_nt_channelwise(a, b, sa, sb, bias, out=out, a_dtype=w.a_fmt, b_dtype=w.b_fmt)
    t = timer.run(fn, steps, warmup)
    t["tflops_kernel"] = 2.0 * M * N * K / (t["kernel_ms_mean"] * 1e-3) / 1e12
    del a, b, sa, sb, bias, out
    return t


def bench_bf16(torch, f, w, steps, warmup, timer):
    """The BF16 comparison path at 4096^3, with torch's BF16 matmul (hipBLASLt)
    on the same operands timed the same way, for context."""
    import numpy as np

    M, N, K = w.shape
    a = torch.from_numpy(w.A.view(np.int16)).cuda().view(torch.bfloat16)
    b = torch.from_numpy(w.B.view(np.int16)).cuda().view(torch.bfloat16)
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    t = timer.run(lambda: f.gemm_nt_bf16(a, b, out=out), steps, warmup)
    t["tflops_kernel"] = 2.0 * M * N * K / (t["kernel_ms_mean"] * 1e-3) / 1e12
    bt = b.t()
    lib = timer.run(lambda: torch.matmul(a, bt, out=out), steps, warmup)
    t["torch_matmul_tflops"] = 2.0 * M * N * K / (lib["kernel_ms_mean"] * 1e-3) / 1e12
    t["torch_matmul_ms_mean"] = lib["kernel_ms_mean"]
    del a, b, bt, out
    return t


def bench_decode(torch, f, M, N, K, steps, warmup, timer, seed=13):
    """Dense few-token GEMM against the HBM roofline: the weights rotate over
    enough copies (> 512 MB in all) that every launch streams them from HBM
    rather than the 256 MB last-level cache."""
    import numpy as np
    import workloads

    w = workloads.dense_random(M, N, K, seed=seed, std=1.0)
    copies = max(2, -(-(512 << 20) // (N * K)))
    base = dev(torch, w.B)
    Bs = [base.roll(i, dims=0).contiguous() for i in range(copies)]
    a = dev(torch, w.A)
    one = torch.ones(1, dtype=torch.float32, device="cuda")
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    # these launches take less than the host's per-call cost: time them from a graph
    t = timer.run_graph(lambda j: f.gemm_nt(a, Bs[j % copies], one, one, out=out, a_dtype=w.a_fmt,
                                            b_dtype=w.b_fmt), copies * max(1, 100 // copies))
    nbytes = float(N * K + M * K + 2 * M * N)
    t["bytes"] = nbytes
    t["gbs_kernel"] = nbytes / (t["kernel_ms_mean"] * 1e-3) / 1e9
    del Bs, base, a, out
    return t


def bench_masked(torch, f, w, steps, warmup, timer):
    import numpy as np

    G, cap, K = w.A.shape
    N = w.B.shape[1]
    a, b = dev(torch, w.A), dev(torch, w.B)
    sa = torch.tensor([w.sa], dtype=torch.float32, device="cuda")
    sb, mm = dev(torch, w.sb), dev(torch, w.masked_m)
    out = torch.empty((G, cap, N), dtype=torch.bfloat16, device="cuda")
    fn = lambda: f.grouped_gemm_masked(a, b, sa, sb, mm, out=out, expected_m=32, a_dtype=w.a_fmt, b_dtype=w.b_fmt)
    t = timer.run(fn, steps, warmup)
    m = np.clip(w.masked_m.astype(np.int64), 0, cap)
    active = int((m > 0).sum())
    # algorithmic bytes: weights of non-empty experts, valid activation rows,
    # valid output rows (BF16), per-expert scales and the counts
    nbytes = active * N * K + int(m.sum()) * K + 2 * int(m.sum()) * N + 4 * G + 4 * (G + 1)
    flops = 2.0 * int(m.sum()) * N * K
    t.update({"bytes": float(nbytes), "flops": flops, "active_experts": active, "valid_rows": int(m.sum()),
              "gbs_wall": nbytes * steps / t["wall_s"] / 1e9,
              "gbs_kernel": nbytes / (t["kernel_ms_mean"] * 1e-3) / 1e9,
              "tflops_kernel": flops / (t["kernel_ms_mean"] * 1e-3) / 1e12})
    del a, b, out
    return t


SWAPAB_TABLE = [(32, 4096, 7168), (96, 4096, 7168), (160, 4096, 7168),
                (32, 7168, 2048), (96, 7168, 2048), (160, 7168, 2048)]


def bench_masked_table(torch, f, steps, warmup, timer, G=16, seed=40):
    """The masked grouped shapes of the swap-AB benchmark table ("One transpose,
    half the compute", section 4): 16 groups, every group m valid rows, the
    kernel the plan picks for that m."""
    import numpy as np
    import workloads

    out = []
    for (n, k) in sorted({(n, k) for _, n, k in SWAPAB_TABLE}):
        cap = max(m for m, nn, kk in SWAPAB_TABLE if (nn, kk) == (n, k))
        w = workloads.masked_random(G, cap, n, k, seed=seed, m_values=[cap] * G)
        a, b, sb = dev(torch, w.A), dev(torch, w.B), dev(torch, w.sb)
        sa = torch.ones(1, dtype=torch.float32, device="cuda")
        o = torch.empty((G, cap, n), dtype=torch.bfloat16, device="cuda")
        for m in sorted(mm for mm, nn, kk in SWAPAB_TABLE if (nn, kk) == (n, k)):
            cnt = torch.full((G,), m, dtype=torch.int32, device="cuda")
            t = timer.run(lambda: f.grouped_gemm_masked(a, b, sa, sb, cnt, out=o, expected_m=m, a_dtype=w.a_fmt,
                                                        b_dtype=w.b_fmt), steps, warmup)
            flops = 2.0 * G * m * n * k
            nbytes = float(G * n * k + G * m * k + 2 * G * m * n)
            ms = t["kernel_ms_mean"]
            out.append({"m": m, "n": n, "k": k, "groups": G, "kernel_us_mean": ms * 1e3, **timing_fields(t),
                        "tflops": flops / (ms * 1e-3) / 1e12, "gbs": nbytes / (ms * 1e-3) / 1e9,
                        "variant": f.plan(1, cap, n, k, G, m).variant})
        del a, b, sb, o, w
    return out


def bench_masked_blockscaled(torch, f, w, steps, warmup, timer):
    import numpy as np

    G, cap, K = w.A.shape
    N = w.B.shape[1]
    a, b = dev(torch, w.A), dev(torch, w.B)
    sa, sb, mm = dev(torch, w.sa), dev(torch, w.sb), dev(torch, w.masked_m)
    out = torch.empty((G, cap, N), dtype=torch.bfloat16, device="cuda")
    fn = lambda: f.grouped_gemm_masked_blockscaled(a, b, sa, sb, mm, out=out, expected_m=32, a_dtype=w.a_fmt,
                                                   b_dtype=w.b_fmt)
    t = timer.run(fn, steps, warmup)
    m = np.clip(w.masked_m.astype(np.int64), 0, cap)
    active = int((m > 0).sum())
    kb, nb = (K + 127) // 128, (N + 127) // 128
    # algorithmic bytes: weights and weight-block scales of non-empty experts,
    # valid token rows and their scales, valid output rows, the counts
    nbytes = active * (N * K + nb * kb) + int(m.sum()) * (K + kb) + 2 * int(m.sum()) * N + 4 * G
    t.update({"bytes": float(nbytes), "gbs_kernel": nbytes / (t["kernel_ms_mean"] * 1e-3) / 1e9})
    del a, b, sa, sb, mm, out
    return t


def bench_contig_blockscaled(torch, f, w, steps, warmup, timer):
    M_total, K = w.A.shape
    G, N, _ = w.B.shape
    a, b = dev(torch, w.A), dev(torch, w.B)
    sa, sb, gi = dev(torch, w.sa), dev(torch, w.sb), dev(torch, w.grp_idx)
    out = torch.empty((M_total, N), dtype=torch.bfloat16, device="cuda")
    fn = lambda: f.grouped_gemm_contig_blockscaled(a, b, sa, sb, gi, out=out, a_dtype=w.a_fmt, b_dtype=w.b_fmt)
    t = timer.run(fn, steps, warmup)
    valid = int((w.grp_idx >= 0).sum())
    t["tflops_kernel"] = 2.0 * valid * N * K / (t["kernel_ms_mean"] * 1e-3) / 1e12
    del a, b, sa, sb, gi, out
    return t


def bench_contig(torch, f, w, steps, warmup, timer):
    M_total, K = w.A.shape
    G, N, _ = w.B.shape
    a, b = dev(torch, w.A), dev(torch, w.B)
    sa = torch.tensor([w.sa], dtype=torch.float32, device="cuda")
    sb, gi = dev(torch, w.sb), dev(torch, w.grp_idx)
    out = torch.empty((M_total, N), dtype=torch.bfloat16, device="cuda")
    fn = lambda: f.grouped_gemm_contig(a, b, sa, sb, gi, out=out, a_dtype=w.a_fmt, b_dtype=w.b_fmt)
    t = timer.run(fn, steps, warmup)
    valid = int((w.grp_idx >= 0).sum())
    flops = 2.0 * valid * N * K
    t.update({"flops": flops, "rows_total": M_total, "rows_valid": valid,
              "tflops_kernel": flops / (t["kernel_ms_mean"] * 1e-3) / 1e12,
              "tflops_wall": flops * steps / t["wall_s"] / 1e12,
              "tflops_kernel_incl_padding": 2.0 * M_total * N * K / (t["kernel_ms_mean"] * 1e-3) / 1e12})
    del a, b, out
    return t


def bench_copy(torch, steps, warmup, timer, nbytes=1 << 30):
    """A plain elementwise copy of known size (fp32 negation: reads nbytes,
    writes nbytes) that calibrates the HBM byte counters."""
    n = nbytes // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    t = timer.run(lambda: torch.neg(src, out=dst), steps, warmup)
    t["bytes_read"] = float(nbytes)
    t["bytes_written"] = float(nbytes)
    t["gbs_kernel"] = 2.0 * nbytes / (t["kernel_ms_mean"] * 1e-3) / 1e9
    del src, dst
    return t


# Kernel-name patterns of the launches each counter summary covers.


# ---------------------------------------------------------------------------
# CPU baseline: the oracle on bounded samples of each configuration.
# ---------------------------------------------------------------------------

def cpu_threads():
    """(threads used, CPUs in this process's affinity): the affinity set,
    capped by OMP_NUM_THREADS where that is set (the CPU share of one GPU)."""
    try:
        aff = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        aff = os.cpu_count() or 1
    omp = int(os.environ.get("OMP_NUM_THREADS", "0") or 0)
    return (min(aff, omp) if omp > 0 else aff), aff


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_dense(w, target_s, label, m_full=None):
    """The oracle on rows 0..R-1 of a dense problem (all columns, full K), R
    sized from a probe so that the pass takes about target_s; a problem that
    takes less than that whole is repeated (at most 20 passes).  w may hold
    only the first rows of A of a problem with m_full rows."""
    import oracle

    threads, _ = cpu_threads()
    M, N, K = w.shape
    r0 = min(M, max(threads, 8))
    t0 = time.perf_counter()
    oracle.gemm_nt(w.A[:r0], w.B, w.a_fmt, w.b_fmt, w.sa, w.sb, threads=threads)
    probe = max(time.perf_counter() - t0, 1e-4)
    rows = int(min(M, max(r0, r0 * target_s / probe)))
    if rows < M:
        rows = max(r0, (rows // threads) * threads)
    passes = 0
    t0 = time.perf_counter()
    while True:
        oracle.gemm_nt(w.A[:rows], w.B, w.a_fmt, w.b_fmt, w.sa, w.sb, threads=threads)
        passes += 1
        el = time.perf_counter() - t0
        if rows < M or el >= 0.67 * target_s or passes >= 20:
            break
    flops = 2.0 * rows * N * K * passes
    mf = m_full or M
    what = (f"rows 0..{rows - 1} of {mf}x{N}x{K} (all {N} columns, full K), {passes} pass(es)" if rows < mf
            else f"the whole {M}x{N}x{K} problem, {passes} pass(es)")
    return {"config": label, "value": flops / el / 1e9, "unit": "GFLOP/s", "cores": threads, "kind": "oracle",
            "seconds": el, "sample": what}


def cpu_masked(w, label):
    """The oracle on the whole masked grouped problem (every valid row)."""
    import numpy as np
    import oracle

    threads, _ = cpu_threads()
    G, cap, K = w.A.shape
    N = w.B.shape[1]
    t0 = time.perf_counter()
    oracle.grouped_masked(w.A, w.B, w.masked_m, w.sb, w.a_fmt, w.b_fmt, w.sa, threads=threads)
    el = time.perf_counter() - t0
    m = np.clip(w.masked_m.astype(np.int64), 0, cap)
    active = int((m > 0).sum())
    nbytes = active * N * K + int(m.sum()) * K + 2 * int(m.sum()) * N + 4 * G + 4 * (G + 1)
    return {"config": label, "value": nbytes / el / 1e9, "unit": "GB/s (algorithmic bytes)",
            "gflops": 2.0 * int(m.sum()) * N * K / el / 1e9, "cores": threads, "kind": "oracle", "seconds": el,
            "sample": f"the whole problem: {int(m.sum())} valid rows over {active} experts"}


def cpu_contig(w, target_s, label, m_full=None):
    """The oracle on the first R rows of the contiguous grouped problem (their
    experts' runs and padding), R sized from a probe; w may hold only the
    first rows of a problem with m_full rows."""
    import numpy as np
    import oracle

    threads, _ = cpu_threads()
    M_total, K = w.A.shape
    G, N, _ = w.B.shape
    r0 = 256
    t0 = time.perf_counter()
    oracle.grouped_contig(w.A[:r0], w.B, w.grp_idx[:r0], w.sb, w.a_fmt, w.b_fmt, w.sa, threads=threads)
    probe = max(time.perf_counter() - t0, 1e-4)
    rows = int(min(M_total, max(r0, r0 * target_s / probe)))
    t0 = time.perf_counter()
    oracle.grouped_contig(w.A[:rows], w.B, w.grp_idx[:rows], w.sb, w.a_fmt, w.b_fmt, w.sa, threads=threads)
    el = time.perf_counter() - t0
    valid = int((w.grp_idx[:rows] >= 0).sum())
    experts = len(np.unique(w.grp_idx[:rows][w.grp_idx[:rows] >= 0]))
    return {"config": label, "value": 2.0 * valid * N * K / el / 1e9, "unit": "GFLOP/s", "cores": threads,
            "kind": "oracle", "seconds": el,
            "sample": f"rows 0..{rows - 1} of {m_full or M_total} ({valid} valid rows over {experts} expert(s))"}


# ---------------------------------------------------------------------------
# Profiling: eager launches for rocprofv3, and the counter summaries.
# ---------------------------------------------------------------------------

# Counter target -> (summary file stem, kernel-name pattern of its dispatches
# in --profile-run, workload, algorithmic FLOPs and bytes per launch or None).
COUNTER_TARGETS = {
    "dense_4096_e4m3": ("tile16_kernel_dense_4096_e4m3", "tile16_kernel<256, 256, 2, 0, 0, 0, 0, false>",
                        "dense 4096^3 E4M3 GEMM (seed 2)"),
    "masked_decode": ("swap_kernel_masked_decode", "swap_kernel<",
                      "masked grouped decode GEMM G=32 cap=64 N=4096 K=7168 m_g~U{0..32} (seed 4)"),
    "contig_prefill": ("ring_kernel_contig_prefill", "ring_kernel<256, 256, 4, 2, 0, 0, 2, 2, 128, 0>",
                       "contiguous grouped prefill GEMM, 65536 routed rows over 32 experts, N=4096 K=7168 (seed 5)"),
    "decode_64": ("decode_kernel_dense_64x4096x7168", "decode_kernel<4, 1, 4, 0, 0, 2, 0, 1>",
                  "dense few-token GEMM M=64 N=4096 K=7168 (seed 13)"),
    "decode_rows_64": ("decode_rows_kernel_dense_64x14336x4096", "decode_rows_kernel<4, 0, 0, 0, 3, 1>",
                       "dense few-token GEMM M=64 N=14336 K=4096, waves on rows (seed 13)"),
    "contig_prefill_blockscaled": ("tile16_kernel_contig_prefill_blockscaled",
                                   "tile16_kernel<256, 256, 2, 0, 0, 2, 1, false>",
                                   "block-scaled contiguous grouped prefill GEMM, 65536 routed rows over 32 experts, "
                                   "N=4096 K=7168 (seed 9)"),
    "dense_4096_bf16": ("ring_kernel_dense_4096_bf16", "ring_kernel<256, 256, 4, 2, 16, 16, 0, 2, 128, 0>",
                        "dense 4096^3 BF16 GEMM, the comparison path (seed 2)"),
}
# Dense matrix-core FLOPs per SIMD per cycle of each target's instruction
# (FP8 by default; BF16 runs at half that rate).
MFMA_FLOPS_PER_CYCLE = {"dense_4096_bf16": 1024.0}
MFMA_COUNT_NOTE = {"dense_4096_bf16": "each 32x32x16 BF16 instruction as 32 cycles, 1024 FLOPs per cycle"}
COPY_PATTERN = "neg_kernel"
PROFILE_LAUNCHES = 6


def profile_run(targets=None):
    """Eager launches of each counter target's workload (all, or those named in
    `targets`) and of the 1 GiB copy that calibrates the byte counters,
    PROFILE_LAUNCHES each, for rocprofv3.  Prints the algorithmic work of each
    target launched as one JSON line."""
    import numpy as np
    import torch

    import fp8_gemm_amd as f
    import workloads

    f.load_library()
    work = {}
    on = lambda name: targets is None or name in targets
    n = 1 << 28
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(PROFILE_LAUNCHES):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst

    if on("dense_4096_e4m3"):
        log("profile: dense 4096^3 E4M3")
        w = workloads.dense_square(workloads.E4M3)
        a, b = dev(torch, w.A), dev(torch, w.B)
        sa = torch.tensor([w.sa], dtype=torch.float32, device="cuda")
        sb = torch.tensor([w.sb], dtype=torch.float32, device="cuda")
        out = torch.empty((4096, 4096), dtype=torch.bfloat16, device="cuda")
        for _ in range(PROFILE_LAUNCHES):
            f.gemm_nt(a, b, sa, sb, out=out, a_dtype=w.a_fmt, b_dtype=w.b_fmt)
        torch.cuda.synchronize()
        fl, by = dense_work(4096, 4096, 4096)
        work["dense_4096_e4m3"] = {"flops": fl, "bytes": by}
        del a, b, out

    if on("dense_4096_bf16"):
        log("profile: dense 4096^3 BF16")
        wb = workloads.dense_bf16_square()
        a = torch.from_numpy(wb.A.view(np.int16)).cuda().view(torch.bfloat16)
        b = torch.from_numpy(wb.B.view(np.int16)).cuda().view(torch.bfloat16)
        out = torch.empty((4096, 4096), dtype=torch.bfloat16, device="cuda")
        for _ in range(PROFILE_LAUNCHES):
            f.gemm_nt_bf16(a, b, out=out)
        torch.cuda.synchronize()
        work["dense_4096_bf16"] = {"flops": 2.0 * 4096 ** 3, "bytes": float(3 * 2 * 4096 * 4096)}
        del a, b, out, wb

    one = torch.ones(1, dtype=torch.float32, device="cuda")
    if on("decode_64"):
        log("profile: dense decode 64x4096x7168")
        wd = workloads.dense_random(64, 4096, 7168, seed=13, std=1.0)
        a, b = dev(torch, wd.A), dev(torch, wd.B)
        out = torch.empty((64, 4096), dtype=torch.bfloat16, device="cuda")
        for _ in range(PROFILE_LAUNCHES):
            f.gemm_nt(a, b, one, one, out=out, a_dtype=wd.a_fmt, b_dtype=wd.b_fmt)
        torch.cuda.synchronize()
        fl, by = dense_work(64, 4096, 7168)
        work["decode_64"] = {"flops": fl, "bytes": by}
        del a, b, out

    if on("decode_rows_64"):
        log("profile: dense decode 64x14336x4096 (waves on rows)")
        wd = workloads.dense_random(64, 14336, 4096, seed=13, std=1.0)
        a, b = dev(torch, wd.A), dev(torch, wd.B)
        out = torch.empty((64, 14336), dtype=torch.bfloat16, device="cuda")
        for _ in range(PROFILE_LAUNCHES):
            f.gemm_nt(a, b, one, one, out=out, a_dtype=wd.a_fmt, b_dtype=wd.b_fmt)
        torch.cuda.synchronize()
        fl, by = dense_work(64, 14336, 4096)
        work["decode_rows_64"] = {"flops": fl, "bytes": by}
        del a, b, out

    if on("masked_decode"):
        log("profile: masked grouped decode")
        wm = workloads.masked_decode()
        G, cap, K = wm.A.shape
        N = wm.B.shape[1]
        a, b = dev(torch, wm.A), dev(torch, wm.B)
        sa = torch.tensor([wm.sa], dtype=torch.float32, device="cuda")
        sb, mm = dev(torch, wm.sb), dev(torch, wm.masked_m)
        out = torch.empty((G, cap, N), dtype=torch.bfloat16, device="cuda")
        for _ in range(PROFILE_LAUNCHES):
            f.grouped_gemm_masked(a, b, sa, sb, mm, out=out, expected_m=32, a_dtype=wm.a_fmt, b_dtype=wm.b_fmt)
        torch.cuda.synchronize()
        m = np.clip(wm.masked_m.astype(np.int64), 0, cap)
        active = int((m > 0).sum())
        work["masked_decode"] = {"flops": 2.0 * int(m.sum()) * N * K,
                                 "bytes": float(active * N * K + int(m.sum()) * K + 2 * int(m.sum()) * N
                                                + 4 * G + 4 * (G + 1))}
        del a, b, out, wm

    if on("contig_prefill"):
        log("profile: contiguous grouped prefill")
        wc = workloads.contig_prefill()
        M_total, K = wc.A.shape
        G, N, _ = wc.B.shape
        a, b = dev(torch, wc.A), dev(torch, wc.B)
        sa = torch.tensor([wc.sa], dtype=torch.float32, device="cuda")
        sb, gi = dev(torch, wc.sb), dev(torch, wc.grp_idx)
        out = torch.empty((M_total, N), dtype=torch.bfloat16, device="cuda")
        for _ in range(PROFILE_LAUNCHES):
            f.grouped_gemm_contig(a, b, sa, sb, gi, out=out, a_dtype=wc.a_fmt, b_dtype=wc.b_fmt)
        torch.cuda.synchronize()
        valid = int((wc.grp_idx >= 0).sum())
        work["contig_prefill"] = {"flops": 2.0 * valid * N * K,
                                  "bytes": float(M_total * K + G * N * K + 2 * valid * N)}
        del a, b, sb, gi, out, wc

    if on("contig_prefill_blockscaled"):
        log("profile: block-scaled contiguous grouped prefill")
        wc = workloads.contig_blockscaled(8192, 8, 32, 4096, 7168, seed=9)
        M_total, K = wc.A.shape
        G, N, _ = wc.B.shape
        a, b = dev(torch, wc.A), dev(torch, wc.B)
        sa, sb, gi = dev(torch, wc.sa), dev(torch, wc.sb), dev(torch, wc.grp_idx)
        out = torch.empty((M_total, N), dtype=torch.bfloat16, device="cuda")
        for _ in range(PROFILE_LAUNCHES):
            f.grouped_gemm_contig_blockscaled(a, b, sa, sb, gi, out=out, a_dtype=wc.a_fmt, b_dtype=wc.b_fmt)
        torch.cuda.synchronize()
        valid = int((wc.grp_idx >= 0).sum())
        work["contig_prefill_blockscaled"] = {"flops": 2.0 * valid * N * K,
                                              "bytes": float(M_total * K + G * N * K + 2 * valid * N
                                                             + wc.sa.nbytes + wc.sb.nbytes)}
        del a, b, sa, sb, gi, out, wc
    print(json.dumps({"profile_run": True, "work": work}), flush=True)


def _csv_files(directory, suffix):
    import glob

    files = glob.glob(os.path.join(directory, "**", f"*{suffix}"), recursive=True)
    if not files:
        raise SystemExit(f"no *{suffix} under {directory}")
    return files


def _counter_rows(directory):
    import csv

    out = {}
    for fpath in _csv_files(directory, "counter_collection.csv"):
        with open(fpath, newline="") as fh:
            for row in csv.DictReader(fh):
                key = (fpath, row["Dispatch_Id"], row["Kernel_Name"])
                out.setdefault(key, {})
                name = row["Counter_Name"]
                out[key][name] = out[key].get(name, 0.0) + float(row["Counter_Value"])
    return out


def _per_dispatch(rows, pattern, counter):
    vals = [c[counter] for (_, d, k), c in rows.items() if pattern in k and counter in c]
    if not vals:
        raise SystemExit(f"no dispatch of a kernel matching {pattern!r} with counter {counter}")
    return sum(vals) / len(vals), len(vals)


def _pmc_durations(directory):
    """{(file, dispatch id, kernel name): seconds} from the start and end
    timestamps a --pmc pass records with each dispatch's counters."""
    import csv

    out = {}
    for fpath in _csv_files(directory, "counter_collection.csv"):
        with open(fpath, newline="") as fh:
            for row in csv.DictReader(fh):
                if "Start_Timestamp" in row and row["Start_Timestamp"]:
                    out[(fpath, row["Dispatch_Id"], row["Kernel_Name"])] = \
                        (int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) * 1e-9
    return out


def _clock_and_busy(rows, durs, pattern):
    """Mean over matching dispatches of the --pmc pass: the kernel's cycles
    (GRBM_GUI_ACTIVE, summed over the 8 XCDs' GRBM blocks, over 8), the clock
    (those cycles over the dispatch's own duration) and the MFMA-busy fraction
    (SQ_VALU_MFMA_BUSY_CYCLES, summed over the 1024 SIMDs, over 1024 x the
    kernel's cycles)."""
    clk, busy, cyc, dur = [], [], [], []
    for key, c in rows.items():
        if pattern not in key[2] or "GRBM_GUI_ACTIVE" not in c or key not in durs:
            continue
        g = c["GRBM_GUI_ACTIVE"] / 8.0
        cyc.append(g)
        dur.append(durs[key])
        clk.append(g / durs[key] / 1e9)
        busy.append(c.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (SIMDS * g) if g else float("nan"))
    n = len(clk)
    if not n:
        raise SystemExit(f"no --pmc dispatch of a kernel matching {pattern!r} with GRBM_GUI_ACTIVE")
    return sum(cyc) / n, sum(dur) / n, sum(clk) / n, sum(busy) / n, n


def _trace_durations(directory, pattern):
    import csv

    durs = []
    for fpath in _csv_files(directory, "kernel_trace.csv"):
        with open(fpath, newline="") as fh:
            for row in csv.DictReader(fh):
                if pattern in row["Kernel_Name"]:
                    durs.append((int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) * 1e-9)
    if not durs:
        raise SystemExit(f"no traced dispatch of a kernel matching {pattern!r}")
    return durs


def pmc_table(dirs, command, out_name):
    """Writes profiles/<out_name>: for each counter target's kernel, the mean
    per dispatch of every counter collected in the given --pmc passes over
    `--profile-run` (one pass per directory), with the derived memory-path
    figures (average L2 read latency seen from the L1, TA cycles per buffer
    instruction)."""
    import csv
    import glob

    vals = {}
    for d in dirs:
        for fpath in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(fpath, newline="") as fh:
                for row in csv.DictReader(fh):
                    for name, (stem, pattern, what) in COUNTER_TARGETS.items():
                        if pattern in row["Kernel_Name"]:
                            key = (name, row["Counter_Name"])
                            disp = (d, row["Dispatch_Id"])     # dispatch ids restart in every pass
                            vals.setdefault(key, {}).setdefault(disp, 0.0)
                            vals[key][disp] += float(row["Counter_Value"])
    lines = ["rocprofv3 --pmc counters per dispatch (mean over dispatches) of the profiled kernels", "",
             "commands (from the repository root R; each pass its own rocprofv3 run over the same program):",
             command, "", f"kernel_source_hash: {kernel_source_hash()}", ""]
    for name, (stem, pattern, what) in COUNTER_TARGETS.items():
        cs = sorted(c for (n, c) in vals if n == name)
        if not cs:
            continue
        lines.append(f"{what} ({pattern}):")
        mean = {c: sum(vals[(name, c)].values()) / len(vals[(name, c)]) for c in cs}
        for c in cs:
            lines.append(f"  {c}: {mean[c]:.0f}")
        if mean.get("TCP_TCC_READ_REQ_sum"):
            lines.append(f"  derived: L2 read latency seen from the L1, mean {mean.get('TCP_TCC_READ_REQ_LATENCY_sum', 0) / mean['TCP_TCC_READ_REQ_sum']:.0f} cycles; "
                         f"{mean['TCP_TCC_READ_REQ_sum'] / 256:.0f} L2 read requests per CU")
        if mean.get("TA_BUFFER_WAVEFRONTS_sum"):
            lines.append(f"  derived: {mean.get('TA_BUFFER_TOTAL_CYCLES_sum', 0) / mean['TA_BUFFER_WAVEFRONTS_sum']:.1f} TA cycles per buffer "
                         f"instruction; {mean.get('TA_BUFFER_TOTAL_CYCLES_sum', 0) / 256:.0f} per CU")
        lines.append("")
    path = os.path.join(PROFILE_DIR, out_name)
    with open(path, "w") as fh:
        fh.write("\n".join(lines))
    log(f"wrote {path}")


def trace_summary(trace_dir, bench_json, command):
    """Writes profiles/bench_kernel_trace.txt from a `rocprofv3 --kernel-trace
    --stats` run of the default bench: rocprofv3's per-kernel statistics, then
    per kernel and grid the dispatch count and mean / median / min duration
    (warm-up and timed launches alike), and beside them the launch durations
    the same bench run measured with its HIP events."""
    import csv
    import gzip
    import glob
    import statistics

    stats = glob.glob(os.path.join(trace_dir, "**", "*kernel_stats.csv"), recursive=True)
    traces = glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv*"), recursive=True)
    if not stats or not traces:
        raise SystemExit(f"no kernel_stats.csv / kernel_trace.csv under {trace_dir}")
    groups = {}
    for fpath in traces:
        opener = gzip.open if fpath.endswith(".gz") else open
        with opener(fpath, "rt", newline="") as fh:
            for row in csv.DictReader(fh):
                name = row["Kernel_Name"]
                if "fp8g::" not in name and "Cijk" not in name:
                    continue
                short = re.sub(r"^void fp8g::|\(fp8g::GemmParams\)$", "", name)
                wg = int(row["Workgroup_Size_X"]) * int(row["Workgroup_Size_Y"]) * int(row["Workgroup_Size_Z"])
                grid = (int(row["Grid_Size_X"]) * int(row["Grid_Size_Y"]) * int(row["Grid_Size_Z"])) // max(wg, 1)
                d = (int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) * 1e-3
                groups.setdefault((short, grid), []).append(d)
    bench = {}
    with open(bench_json) as fh:
        for line in fh:
            if line.startswith("{") and '"metric"' in line:
                bench = json.loads(line)
    lines = [
        "rocprofv3 kernel trace of the default benchmark run (every leg; warm-up launches included)",
        "",
        "command (on the GPU host, from the repository root R):",
        command,
        "",
        f"kernel_source_hash: {kernel_source_hash()}",
        "",
        "kernel_stats.csv (rocprofv3 --stats):",
    ]
    with open(stats[0]) as fh:
        for row in csv.reader(fh):
            if row[0] == "Name" or "fp8g::" in row[0] or "Cijk" in row[0]:
                lines.append(",".join(row[:7]))
    lines += ["", "per kernel and grid (workgroups): dispatches, mean / median / min duration in us"]
    for (short, grid), ds in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"  {short:60s} grid {grid:6d}: {len(ds):6d}  {statistics.mean(ds):10.2f} "
                     f"{statistics.median(ds):10.2f} {min(ds):10.2f}")
    if bench:
        r = bench["roofline"]
        lines += ["", "the same run's HIP-event figures (bench.py's JSON line):",
                  f"  dense 4096^3 E4M3 (tile16_kernel<256, 256, 2, 0, 0, 0, 0, false>, grid 256): "
                  f"mean {r['kernel_ms_mean'] * 1e3:.2f} us, median {r['us_median']:.2f} us, "
                  f"{r['achieved']:.0f} TFLOP/s"]
        for key, label in (("dense_4096_e5m2", "dense 4096^3 E5M2"), ("dense_4096_blockscaled", "block-scaled 4096^3"),
                           ("dense_4096_channelwise", "per-channel 4096^3"), ("masked_grouped", "masked decode"),
                           ("masked_grouped_blockscaled", "block-scaled masked decode"),
                           ("contig_grouped", "contiguous prefill"),
                           ("contig_grouped_blockscaled", "block-scaled contiguous prefill")):
            if key in bench:
                lines.append(f"  {label}: mean {bench[key]['kernel_ms_mean'] * 1e3:.2f} us, "
                             f"median {bench[key]['us_median']:.2f} us")
    path = os.path.join(PROFILE_DIR, "bench_kernel_trace.txt")
    with open(path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    log(f"wrote {path}")


SQ_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CYCLES", "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE",
               "SQ_INSTS_LDS", "SQ_INSTS_VALU", "SQ_INSTS_SALU", "GRBM_GUI_ACTIVE", "GRBM_COUNT")


def counters_summary(trace_dir, fetch_dir, write_dir, sq_dir, command, work_json):
    """Writes profiles/<kernel>_<workload>_counters.txt for every counter target
    from a --kernel-trace pass and three --pmc passes over `--profile-run`."""
    import statistics

    work = json.loads(work_json)["work"] if work_json else {}
    fr, wr, sr = _counter_rows(fetch_dir), _counter_rows(write_dir), _counter_rows(sq_dir)
    sq_durs = _pmc_durations(sq_dir)
    copy_cyc, copy_dur, copy_clk, _, _ = _clock_and_busy(sr, sq_durs, COPY_PATTERN)
    copy_f, ncf = _per_dispatch(fr, COPY_PATTERN, "FETCH_SIZE")
    copy_w, ncw = _per_dispatch(wr, COPY_PATTERN, "WRITE_SIZE")
    nbytes = float(1 << 30)
    kf, kw = nbytes / (copy_f * 1024.0), nbytes / (copy_w * 1024.0)
    h = kernel_source_hash()
    for name, (stem, pattern, what) in COUNTER_TARGETS.items():
        if work and name not in work:
            continue                # not launched by this --profile-run
        durs = _trace_durations(trace_dir, pattern)
        dur = statistics.mean(durs)
        f_kib, nf = _per_dispatch(fr, pattern, "FETCH_SIZE")
        w_kib, nw = _per_dispatch(wr, pattern, "WRITE_SIZE")
        rd, wt = f_kib * 1024.0 * kf, w_kib * 1024.0 * kw
        sq = {}
        for c in SQ_COUNTERS:
            sq[c] = _per_dispatch(sr, pattern, c)[0]
        cyc, pmc_dur, clock, mfma_busy, npmc = _clock_and_busy(sr, sq_durs, pattern)
        # GRBM_GUI_ACTIVE counts the whole collection window; for a dispatch of
        # a few microseconds that window is longer than the kernel, and the
        # ratio reads above any clock the part runs at
        clock_ok = clock <= 1.05 * copy_clk
        w = work.get(name, {})
        lines = [
            f"rocprofv3 counters: {what}",
            "",
            "commands (from the repository root; each pass its own rocprofv3 run over the same program):",
            command,
            "",
            f"kernel_source_hash: {h}",
            f"kernel name pattern: {pattern}",
            f"dispatches: trace {len(durs)}, FETCH {nf}, WRITE {nw}, SQ/GRBM {_per_dispatch(sr, pattern, 'GRBM_GUI_ACTIVE')[1]}",
            f"kernel duration (trace pass, mean over dispatches): {dur * 1e6:.2f} us "
            f"(min {min(durs) * 1e6:.2f}, max {max(durs) * 1e6:.2f})",
            "",
            "HBM traffic (FETCH_SIZE / WRITE_SIZE passes):",
            f"  FETCH_SIZE per dispatch: {f_kib:.1f} KiB; WRITE_SIZE per dispatch: {w_kib:.1f} KiB",
            f"  calibration, fp32 negation of 1 GiB (reads 1 GiB, writes 1 GiB), {ncf}/{ncw} dispatches: "
            f"FETCH_SIZE {copy_f:.1f} KiB -> read factor {kf:.4f}; WRITE_SIZE {copy_w:.1f} KiB -> write factor {kw:.4f}",
            f"  hbm_read_bytes_per_launch: {rd:.0f}",
            f"  hbm_write_bytes_per_launch: {wt:.0f}",
            f"  hbm_bytes_per_launch: {rd + wt:.0f}",
        ]
        if w:
            lines += [f"  algorithmic_bytes_per_launch: {w['bytes']:.0f}  (traffic / algorithmic = {(rd + wt) / w['bytes']:.3f})",
                      f"  algorithmic_flops_per_launch: {w['flops']:.0f}",
                      f"  achieved over the traced duration: {w['flops'] / dur / 1e12:.1f} TFLOP/s, "
                      f"{w['bytes'] / dur / 1e9:.0f} GB/s algorithmic, {(rd + wt) / dur / 1e9:.0f} GB/s counted"]
        lines += [
            "",
            "SQ / GRBM pass (values per dispatch, summed over the counter's instances):",
        ] + [f"  {c}: {sq[c]:.0f}" for c in SQ_COUNTERS] + [
            "",
            f"derived (SQ / GRBM pass, {npmc} dispatches, their own timestamps; counter collection serialises "
            "the launches and lengthens them):",
            f"  dispatch duration in this pass: {pmc_dur * 1e6:.2f} us",
            f"  kernel cycles (GRBM_GUI_ACTIVE / 8 XCDs): {cyc:.0f}",
            (f"  effective_clock_ghz: {clock:.3f}  (kernel cycles / dispatch duration; the memory-bound 1 GiB copy "
             f"reads {copy_clk:.3f} GHz the same way)") if clock_ok else
            (f"  effective clock: not measurable ({clock:.3f} GHz from the ratio, above the copy's {copy_clk:.3f}: "
             f"the counter window is longer than this short dispatch)"),
            (f"  mfma_busy_fraction: {mfma_busy:.4f}  (SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x kernel cycles); the "
             f"counter counts {MFMA_COUNT_NOTE.get(name, 'each 16x16x128 FP8 instruction as 32 cycles')})") if clock_ok else
            (f"  MFMA busy: at most {mfma_busy:.4f} of the counter window (SQ_VALU_MFMA_BUSY_CYCLES / "
             f"(1024 SIMDs x window cycles))"),
            f"  lds_bank_conflict_fraction: {sq['SQ_LDS_BANK_CONFLICT'] / sq['SQ_LDS_IDX_ACTIVE'] if sq['SQ_LDS_IDX_ACTIVE'] else 0.0:.4f}"
            f"  (SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE)",
        ]
        if w.get("flops") and clock_ok:
            rate = MFMA_FLOPS_PER_CYCLE.get(name, 2048.0)
            lines.append(f"  MFMA-bound time at the effective clock: {w['flops'] / (SIMDS * rate * clock * 1e9) * 1e6:.2f} us "
                         f"(against {dur * 1e6:.2f} us traced)")
        path = os.path.join(PROFILE_DIR, f"{stem}_counters.txt")
        with open(path, "w") as fh:
            fh.write("\n".join(lines) + "\n")
        log(f"wrote {path}")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--only", nargs="*", default=None,
                    help="subset of: dense masked masked_table masked_bs contig contig_bs small e5m2 blockscaled "
                         "channelwise bf16 decode proj copy (default: all)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--profile-run", action="store_true",
                    help="eager launches of the counter targets' workloads, for rocprofv3 (no timing)")
    ap.add_argument("--profile-targets", nargs="+", default=None, choices=sorted(COUNTER_TARGETS),
                    help="with --profile-run: only these counter targets (default: all)")
    ap.add_argument("--counters-summary", nargs=4, metavar=("TRACE_DIR", "FETCH_DIR", "WRITE_DIR", "SQ_DIR"),
                    default=None, help="write profiles/*_counters.txt from rocprofv3 output directories (no GPU work)")
    ap.add_argument("--counters-command", default="",
                    help="the commands that produced the counter directories (recorded in the summaries)")
    ap.add_argument("--counters-work", default="", help="the JSON line --profile-run printed")
    ap.add_argument("--pmc-table", nargs="+", metavar="PMC_DIR",
                    help="write profiles/memory_path_counters.txt from --pmc passes over --profile-run")
    ap.add_argument("--trace-summary", nargs=2, metavar=("TRACE_DIR", "BENCH_JSON"),
                    help="write profiles/bench_kernel_trace.txt from a --kernel-trace --stats run of the bench")
    args = ap.parse_args()

    if args.counters_summary:
        counters_summary(*args.counters_summary, args.counters_command, args.counters_work)
        return
    if args.trace_summary:
        trace_summary(*args.trace_summary, args.counters_command)
        return
    if args.pmc_table:
        pmc_table(args.pmc_table, args.counters_command, "memory_path_counters.txt")
        return

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the FP8 GEMM path has no multi-GPU component)", file=sys.stderr)
        sys.exit(2)

    import torch

    import fp8_gemm_amd as f
    import workloads

    f.load_library()
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.profile_run:
        profile_run(args.profile_targets)
        return
    timer = Timer(torch)
    want = set(args.only) if args.only else {"dense", "masked", "masked_table", "masked_bs", "contig", "contig_bs",
                                           "small", "e5m2", "blockscaled", "channelwise", "bf16", "decode", "proj",
                                           "copy"}
    steps, warmup = args.steps, args.warmup
    extra = {}
    cpu_jobs = []           # oracle samples, run after every GPU leg

    log("generating dense 4096^3 E4M3 inputs")
    wd = workloads.dense_square(workloads.E4M3)
    dense = None
    if "dense" in want:
        log("timing dense 4096^3 E4M3")
        dense = bench_dense(torch, f, wd, steps, warmup, timer)
        log(f"  {dense['tflops_kernel']:.1f} TFLOP/s per launch, {dense['tflops_wall']:.1f} whole-job; "
            f"median {dense['median_ms'] * 1e3:.2f} us (p10 {dense['p10_ms'] * 1e3:.2f}, p90 {dense['p90_ms'] * 1e3:.2f})")
        cpu_jobs.append(lambda: cpu_dense(wd, 6.0, "dense 4096^3 E4M3"))
    if "e5m2" in want:
        log("timing dense 4096^3 E5M2")
        w5 = workloads.dense_square(workloads.E5M2)
        r = bench_dense(torch, f, w5, steps, warmup, timer)
        extra["dense_4096_e5m2"] = {"tflops_kernel": r["tflops_kernel"], "tflops_wall": r["tflops_wall"],
                                    "kernel_ms_mean": r["kernel_ms_mean"],
                                    "frac_of_peak": r["tflops_kernel"] / PEAK_FP8_TFLOPS, **timing_fields(r)}
        w5s = workloads.Dense(w5.A[:1024].copy(), w5.B, w5.sa, w5.sb, w5.a_fmt, w5.b_fmt, w5.name)
        cpu_jobs.append(lambda: cpu_dense(w5s, 2.0, "dense 4096^3 E5M2", m_full=4096))
        del w5
    if "blockscaled" in want:
        log("timing block-scaled dense 4096^3 E4M3 (power-of-two scales per 1x128 / 128x128 block)")
        wbs = workloads.dense_blockscaled_square()
        r = bench_blockscaled(torch, f, wbs, steps, warmup, timer)
        extra["dense_4096_blockscaled"] = {
            "workload": "dense 4096^3 E4M3, activations N(0,1) per 1x128 block and weights N(0,0.02) per "
                        "128x128 block, each with its own power-of-two (E8M0) scale (seed 6)",
            "tflops_kernel": r["tflops_kernel"], "kernel_ms_mean": r["kernel_ms_mean"],
            "frac_of_peak": r["tflops_kernel"] / PEAK_FP8_TFLOPS, **timing_fields(r)}
        log(f"  {r['tflops_kernel']:.1f} TFLOP/s")
        del wbs
    if "channelwise" in want:
        log("timing dense 4096^3 E4M3 with per-row / per-channel scales and a per-channel bias")
        r = bench_channelwise(torch, f, wd, steps, warmup, timer)
        extra["dense_4096_channelwise"] = {
            "workload": "dense 4096^3 E4M3 (seed 2 operands), row scales and channel scales U[0.5,2], "
                        "bias N(0,1), applied in the epilogue",
            "tflops_kernel": r["tflops_kernel"], "kernel_ms_mean": r["kernel_ms_mean"],
            "frac_of_peak": r["tflops_kernel"] / PEAK_FP8_TFLOPS, **timing_fields(r)}
        log(f"  {r['tflops_kernel']:.1f} TFLOP/s")
    if "bf16" in want:
        log("timing the BF16 comparison path, 4096^3")
        wb = workloads.dense_bf16_square()
        r = bench_bf16(torch, f, wb, steps, warmup, timer)
        extra["dense_4096_bf16"] = {
            "workload": "BF16 comparison GEMM 4096^3, the seed-2 draws of the FP8 case rounded to BF16, no scales",
            "tflops_kernel": r["tflops_kernel"], "kernel_ms_mean": r["kernel_ms_mean"], **timing_fields(r),
            "roofline": {"bound": "mfma", "achieved": r["tflops_kernel"], "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": r["tflops_kernel"] / PEAK_BF16_TFLOPS},
            "context_torch_matmul": {"tflops": r["torch_matmul_tflops"], "ms_mean": r["torch_matmul_ms_mean"]}}
        log(f"  {r['tflops_kernel']:.1f} TFLOP/s (torch.matmul {r['torch_matmul_tflops']:.1f})")
        del wb
    if "decode" in want:
        out = []
        for (N, K, Ms) in ((4096, 7168, (1, 16, 32, 64)), (14336, 4096, (1, 16, 32, 64)), (2048, 7168, (1, 64))):
            for M in Ms:
                r = bench_decode(torch, f, M, N, K, steps, warmup, timer)
                out.append({"M": M, "N": N, "K": K, "kernel_us_mean": r["kernel_ms_mean"] * 1e3, **timing_fields(r),
                            "variant": f.plan(0, M, N, K).variant, "k_splits": f.plan(0, M, N, K).k_splits,
                            "rows_per_workgroup": f.plan(0, M, N, K).tile_n,
                            "roofline": {"bound": "hbm", "achieved": r["gbs_kernel"], "peak": PEAK_HBM_GBS,
                                         "unit": "GB/s", "frac": r["gbs_kernel"] / PEAK_HBM_GBS,
                                         "algorithmic_bytes": r["bytes"]}})
                log(f"  decode {M}x{N}x{K}: {r['kernel_ms_mean'] * 1e3:.2f} us, {r['gbs_kernel']:.0f} GB/s")
        extra["dense_decode"] = {
            "workload": "dense few-token GEMMs, A ~N(0,1), B ~N(0,1) E4M3 (seed 13), weights rotated over "
                        "> 512 MB of copies so each launch reads them from HBM",
            "timing": "launches captured in a graph and replayed (eager calls through Python cost ~10 us each); "
                      "median/p10/p90 per replay",
            "shapes": out}
    if "small" in want:
        log("timing dense 256^3")
        ws = workloads.dense_small()
        r = bench_dense(torch, f, ws, steps, warmup, timer)
        a, b = dev(torch, ws.A), dev(torch, ws.B)
        one = torch.ones(1, dtype=torch.float32, device="cuda")
        o = torch.empty((256, 256), dtype=torch.bfloat16, device="cuda")
        g = timer.run_graph(lambda j: f.gemm_nt(a, b, one, one, out=o, a_dtype=ws.a_fmt, b_dtype=ws.b_fmt), 100)
        extra["dense_256"] = {"kernel_us_mean": r["kernel_ms_mean"] * 1e3,
                              "us_per_call_wall": r["wall_s"] / steps * 1e6, "bound": "launch latency",
                              "kernel_us_graph": g["kernel_ms_mean"] * 1e3, "graph": timing_fields(g),
                              "eager": timing_fields(r), "variant": f.plan(0, 256, 256, 256).variant}
        cpu_jobs.append(lambda: cpu_dense(ws, 0.5, "dense 256^3"))
        del a, b, o
    if "masked" in want:
        log("generating masked grouped decode inputs (G=32, cap=64, N=4096, K=7168)")
        wm = workloads.masked_decode()
        log("timing masked grouped decode")
        r = bench_masked(torch, f, wm, steps, warmup, timer)
        ctr = read_counters("masked_decode")
        extra["masked_grouped"] = {
            "workload": "masked grouped FP8 GEMM, G=32, cap=64, N=4096, K=7168, m_g~U{0..32} (seed 4), E4M3, swap-AB",
            "gbs_kernel": r["gbs_kernel"], "gbs_wall": r["gbs_wall"], "kernel_ms_mean": r["kernel_ms_mean"],
            **timing_fields(r),
            "tflops_kernel": r["tflops_kernel"], "active_experts": r["active_experts"], "valid_rows": r["valid_rows"],
            "roofline": {"bound": "hbm", "achieved": r["gbs_kernel"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": r["gbs_kernel"] / PEAK_HBM_GBS,
                         "traffic": ctr.get("hbm_bytes_per_launch") if ctr else None,
                         "algorithmic_bytes": r["bytes"]}}
        log(f"  {r['gbs_kernel']:.0f} GB/s ({r['gbs_kernel'] / PEAK_HBM_GBS:.1%} of HBM peak)")
        cpu_jobs.append(lambda: cpu_masked(wm, "masked grouped decode G=32 cap=64 N=4096 K=7168"))
    if "masked_table" in want:
        log("timing the swap-AB benchmark table shapes (16 groups, m in {32, 96, 160})")
        rows = bench_masked_table(torch, f, max(10, steps // 4), max(2, warmup // 4), timer)
        extra["masked_swapab_table"] = {
            "workload": "masked grouped FP8 GEMM, 16 groups, every group m rows, (n, k) in {(4096, 7168), "
                        "(7168, 2048)}, E4M3, weights amax-scaled N(0,0.02) (seed 40)", "shapes": rows}
        for r in rows:
            log(f"  m={r['m']} n={r['n']} k={r['k']}: {r['kernel_us_mean']:.1f} us, {r['tflops']:.0f} TFLOP/s, "
                f"{r['gbs']:.0f} GB/s")
    if "masked_bs" in want:
        log("generating block-scaled masked grouped decode inputs (G=32, cap=64, N=4096, K=7168)")
        wmb = workloads.masked_decode_blockscaled()
        r = bench_masked_blockscaled(torch, f, wmb, steps, warmup, timer)
        extra["masked_grouped_blockscaled"] = {
            "workload": "block-scaled masked grouped FP8 GEMM, G=32, cap=64, N=4096, K=7168, m_g~U{0..32} (seed 8), "
                        "E8M0 scales per 1x128 token block and 128x128 weight block, swap-AB",
            "kernel_ms_mean": r["kernel_ms_mean"], **timing_fields(r),
            "roofline": {"bound": "hbm", "achieved": r["gbs_kernel"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": r["gbs_kernel"] / PEAK_HBM_GBS, "algorithmic_bytes": r["bytes"]}}
        log(f"  {r['gbs_kernel']:.0f} GB/s")
        del wmb
    if "contig" in want:
        log("generating contiguous grouped prefill inputs (65536 rows over 32 experts, N=4096, K=7168)")
        wc = workloads.contig_prefill()
        log("timing contiguous grouped prefill")
        r = bench_contig(torch, f, wc, max(5, steps // 5), max(2, warmup // 5), timer)
        extra["contig_grouped"] = {
            "workload": "contiguous grouped FP8 GEMM, 8192 tokens x top-8 over 32 experts, N=4096, K=7168 (seed 5)",
            "tflops_kernel": r["tflops_kernel"], "tflops_wall": r["tflops_wall"],
            "frac_of_peak": r["tflops_kernel"] / PEAK_FP8_TFLOPS, "kernel_ms_mean": r["kernel_ms_mean"],
            **timing_fields(r),
            "rows_total": r["rows_total"], "rows_valid": r["rows_valid"],
            "tflops_kernel_incl_padding": r["tflops_kernel_incl_padding"]}
        log(f"  {r['tflops_kernel']:.1f} TFLOP/s")
        wcs = workloads.Contig(A=wc.A[:4096].copy(), B=wc.B, grp_idx=wc.grp_idx[:4096].copy(), sa=wc.sa, sb=wc.sb,
                               a_fmt=wc.a_fmt, b_fmt=wc.b_fmt, name=wc.name)
        mt = wc.A.shape[0]
        cpu_jobs.append(lambda: cpu_contig(wcs, 3.0, "contiguous grouped prefill 65536 rows, N=4096 K=7168", m_full=mt))
        del wc
    if "contig_bs" in want:
        log("generating block-scaled contiguous grouped prefill inputs")
        wcb = workloads.contig_blockscaled(8192, 8, 32, 4096, 7168, seed=9)
        r = bench_contig_blockscaled(torch, f, wcb, max(5, steps // 5), max(2, warmup // 5), timer)
        extra["contig_grouped_blockscaled"] = {
            "workload": "block-scaled contiguous grouped FP8 GEMM, 8192 tokens x top-8 over 32 experts, N=4096, "
                        "K=7168, E8M0 scales per 1x128 token block and 128x128 weight block (seed 9)",
            "tflops_kernel": r["tflops_kernel"], "kernel_ms_mean": r["kernel_ms_mean"], **timing_fields(r),
            "frac_of_peak": r["tflops_kernel"] / PEAK_FP8_TFLOPS}
        log(f"  {r['tflops_kernel']:.1f} TFLOP/s")
        del wcb
    if "proj" in want:
        out = []
        for i in range(len(workloads.PROJECTION_SHAPES)):
            wp = workloads.projection(i)
            r = bench_dense(torch, f, wp, max(5, steps // 2), max(2, warmup // 2), timer)
            M, N, K = wp.shape
            out.append({"M": M, "N": N, "K": K, "tflops_kernel": r["tflops_kernel"],
                        "frac_of_peak": r["tflops_kernel"] / PEAK_FP8_TFLOPS, "kernel_ms_mean": r["kernel_ms_mean"],
                        **timing_fields(r), "variant": f.plan(0, M, N, K).variant})
            log(f"  projection {M}x{N}x{K}: {r['tflops_kernel']:.1f} TFLOP/s")
            wps = workloads.Dense(wp.A[:256].copy(), wp.B, wp.sa, wp.sb, wp.a_fmt, wp.b_fmt, wp.name)
            cpu_jobs.append(lambda wps=wps, M=M, N=N, K=K: cpu_dense(wps, 1.0, f"projection {M}x{N}x{K}", m_full=M))
            del wp
        extra["projections"] = out

    if "copy" in want:
        log("timing the 1 GiB copy used to calibrate the HBM byte counters")
        r = bench_copy(torch, steps, warmup, timer)
        extra["copy_1gib"] = {"gbs_kernel": r["gbs_kernel"], "kernel_ms_mean": r["kernel_ms_mean"]}
        log(f"  {r['gbs_kernel']:.0f} GB/s read+write")

    cpu = None
    if not args.no_cpu and cpu_jobs:
        threads, aff = cpu_threads()
        log(f"timing the CPU oracle on samples of {len(cpu_jobs)} configurations ({threads} threads)")
        per_config = []
        for job in cpu_jobs:
            res = job()
            log(f"  {res['config']}: {res['value']:.2f} {res['unit']} over {res['seconds']:.1f} s ({res['sample']})")
            per_config.append(res)
        head = per_config[0] if dense is not None else None
        cpu = {"value": head["value"] / 1e3 if head else None, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
               "sample": (f"{head['sample']} of the dense 4096^3 E4M3 problem, {head['seconds']:.1f} s on {threads} "
                          f"host threads" if head else None),
               "affinity_cpus": aff, "cpu_model": cpu_model(),
               "threads_note": "the process's CPU affinity, capped by OMP_NUM_THREADS where set",
               "per_config": per_config}

    if dense is None:
        print(json.dumps({"metric": METRIC, "partial": True, "cpu_baseline": cpu, **extra}))
        return
    ctr = read_counters("dense_4096_e4m3")
    line = {
        "metric": METRIC,
        "value": dense["tflops_wall"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": dense["wall_s"] / steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3",
        "data": "synthetic",
        "config": {"workload": "dense FP8 GEMM D=A.B^T, M=N=K=4096, E4M3 A and B (K-major), "
                               "entries N(0,1)*0.5, per-tensor scales U[0.5,2], FP32 accumulate, BF16 out (seed 2)",
                   "M": 4096, "N": 4096, "K": 4096},
        "roofline": {"bound": "mfma", "achieved": dense["tflops_kernel"], "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                     "frac": dense["tflops_kernel"] / PEAK_FP8_TFLOPS,
                     "traffic": ctr.get("hbm_bytes_per_launch") if ctr else None,
                     "kernel_ms_mean": dense["kernel_ms_mean"], **timing_fields(dense),
                     "mfma_busy_fraction": ctr.get("mfma_busy_fraction") if ctr else None,
                     "effective_clock_ghz": ctr.get("effective_clock_ghz") if ctr else None,
                     "algorithmic_flops": dense["flops"], "algorithmic_bytes": dense["bytes"]},
        "cpu_baseline": cpu,
        "kernel_source_hash": kernel_source_hash(),
    }
    line.update(extra)
    print(json.dumps(line))


if __name__ == "__main__":
    main()
