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

The average launch duration of each leg is the interval between two HIP events
recorded around its K back-to-back launches on the stream the kernels run on
(torch's current stream, which the library is handed), divided by K.  The CPU
baseline is the oracle, timed on a bounded sample of the dense 4096^3 problem
(whole-problem passes until about 10-15 s have passed).  The 1 GiB copy leg
calibrates the rocprofv3 HBM byte counters (--counters-summary).

    python bench.py [--gpus 1] [--steps 200] [--warmup 20] [--only NAME ...] [--no-cpu]
    python bench.py --counters-summary FETCH_DIR WRITE_DIR --counters-command "..."
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP8_TFLOPS = 5000.0      # MI355X dense FP8 matrix peak (no sparsity)
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense BF16 matrix peak (no sparsity)
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


def read_traffic(name: str):
    """HBM bytes per launch recorded from rocprofv3 counters for `name`, or None
    when no summary exists or the kernels changed since it was taken."""
    path = os.path.join(PROFILE_DIR, f"{name}_hbm_counters.txt")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"kernel_source_hash:\s*(\w+)", text)
    m_bytes = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_hash or not m_bytes or m_hash.group(1) != kernel_source_hash():
        return None
    return float(m_bytes.group(1))


class Timer:
    """Times `fn` (which launches work on torch's current stream): at least
    `warmup` untimed calls and at least `min_warm_s` seconds of them (the GPU
    clock ramps up over the first few milliseconds of load after idle), then
    exactly `steps` back-to-back calls between one pair of HIP events recorded
    on that stream, with a synchronize on both sides of the timed region.  The
    average launch duration is the event interval over `steps`."""

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
        return {"wall_s": wall, "kernel_ms_mean": e0.elapsed_time(e1) / steps, "warmup_calls": done}

    def run_graph(self, fn, n, replays=5):
        """For launches shorter than the host's per-call cost (~10 us through
        Python): fn(j) for j < n captured once in a graph, which is replayed
        for at least `min_warm_s` seconds, then `replays` times between one
        pair of events on the replay stream.  The average launch duration is
        the event interval over replays * n."""
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
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(replays):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        del g
        return {"kernel_ms_mean": e0.elapsed_time(e1) / (replays * n), "launches": replays * n}


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
            out.append({"m": m, "n": n, "k": k, "groups": G, "kernel_us_mean": ms * 1e3,
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


def cpu_baseline(w, target_s=15.0, max_passes=20):
    """The oracle on the dense problem: rows 0..R-1 (all columns, full K), R
    chosen so one pass takes about target_s seconds; when the whole problem
    takes less than that, whole-problem passes are repeated until about
    target_s seconds have passed (at most max_passes)."""
    import oracle

    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or oracle.default_threads()
    threads = max(1, min(threads, oracle.default_threads(), 16))
    M, N, K = w.shape
    r0 = 8
    t0 = time.perf_counter()
    oracle.gemm_nt(w.A[:r0], w.B, w.a_fmt, w.b_fmt, w.sa, w.sb, threads=threads)
    probe = time.perf_counter() - t0
    rows = int(min(M, max(threads, r0 * target_s / max(probe, 1e-3))))
    rows = M if rows >= M else max(threads, (rows // threads) * threads)
    passes = 0
    t0 = time.perf_counter()
    while True:
        oracle.gemm_nt(w.A[:rows], w.B, w.a_fmt, w.b_fmt, w.sa, w.sb, threads=threads)
        passes += 1
        el = time.perf_counter() - t0
        if rows < M or el >= 0.67 * target_s or passes >= max_passes:
            break
    flops = 2.0 * rows * N * K * passes
    what = (f"rows 0..{rows - 1} of the {M}x{N}x{K} E4M3 problem (all {N} columns, full K)" if rows < M
            else f"the whole {M}x{N}x{K} E4M3 problem, {passes} pass(es)")
    return {"value": flops / el / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{what}, {el:.1f} s on {threads} host threads", "seconds": el}


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
COUNTER_TARGETS = {
    "dense_4096_e4m3": ("tile16_kernel<256, 256, 2, 0, 0, 0, 0,", "dense 4096^3 E4M3 GEMM"),
    "masked_decode": ("swap_kernel<", "masked grouped decode GEMM G=32 cap=64 N=4096 K=7168 m_g~U{0..32}"),
}
COPY_PATTERN = "neg_kernel"


def _counter_rows(directory):
    import csv
    import glob

    files = glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no *counter_collection.csv under {directory}")
    out = {}
    for fpath in files:
        with open(fpath, newline="") as fh:
            for row in csv.DictReader(fh):
                key = (row["Dispatch_Id"], row["Kernel_Name"])
                out.setdefault(key, {})
                name = row["Counter_Name"]
                out[key][name] = out[key].get(name, 0.0) + float(row["Counter_Value"])
    return out


def _per_dispatch(rows, pattern, counter):
    vals = [c[counter] for (d, k), c in rows.items() if pattern in k and counter in c]
    if not vals:
        raise SystemExit(f"no dispatch of a kernel matching {pattern!r} with counter {counter}")
    return sum(vals) / len(vals), len(vals)


def counters_summary(fetch_dir, write_dir, command):
    """Writes profiles/<name>_hbm_counters.txt from a rocprofv3 --pmc FETCH_SIZE
    run and a --pmc WRITE_SIZE run (KiB per dispatch), each scaled by what the
    same counter reads for the copy kernel of known size."""
    fr, wr = _counter_rows(fetch_dir), _counter_rows(write_dir)
    copy_f, ncf = _per_dispatch(fr, COPY_PATTERN, "FETCH_SIZE")
    copy_w, ncw = _per_dispatch(wr, COPY_PATTERN, "WRITE_SIZE")
    nbytes = float(1 << 30)
    kf, kw = nbytes / (copy_f * 1024.0), nbytes / (copy_w * 1024.0)
    h = kernel_source_hash()
    for name, (pattern, what) in COUNTER_TARGETS.items():
        f_kib, nf = _per_dispatch(fr, pattern, "FETCH_SIZE")
        w_kib, nw = _per_dispatch(wr, pattern, "WRITE_SIZE")
        rd, wt = f_kib * 1024.0 * kf, w_kib * 1024.0 * kw
        text = (f"rocprofv3 HBM byte counters: {what}\n\n"
                f"commands (from the repository root):\n{command}\n\n"
                f"kernel_source_hash: {h}\n"
                f"kernel name pattern: {pattern}  (dispatches: FETCH {nf}, WRITE {nw})\n"
                f"FETCH_SIZE per dispatch: {f_kib:.1f} KiB\n"
                f"WRITE_SIZE per dispatch: {w_kib:.1f} KiB\n"
                f"calibration, fp32 negation of 1 GiB (reads 1 GiB, writes 1 GiB), {ncf}/{ncw} dispatches:\n"
                f"  FETCH_SIZE {copy_f:.1f} KiB -> read factor {kf:.4f}\n"
                f"  WRITE_SIZE {copy_w:.1f} KiB -> write factor {kw:.4f}\n"
                f"hbm_read_bytes_per_launch: {rd:.0f}\n"
                f"hbm_write_bytes_per_launch: {wt:.0f}\n"
                f"hbm_bytes_per_launch: {rd + wt:.0f}\n")
        path = os.path.join(PROFILE_DIR, f"{name}_hbm_counters.txt")
        with open(path, "w") as fh:
            fh.write(text)
        log(f"wrote {path}: {(rd + wt) / 1e6:.1f} MB per launch")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--only", nargs="*", default=None,
                    help="subset of: dense masked masked_table masked_bs contig contig_bs small e5m2 blockscaled channelwise bf16 decode "
                         "proj copy "
                         "(default: all)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--counters-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"), default=None,
                    help="write profiles/*_hbm_counters.txt from rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE "
                         "output directories (no GPU work)")
    ap.add_argument("--counters-command", default="",
                    help="the commands that produced the counter directories (recorded in the summary)")
    args = ap.parse_args()

    if args.counters_summary:
        counters_summary(args.counters_summary[0], args.counters_summary[1], args.counters_command)
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
    timer = Timer(torch)
    want = set(args.only) if args.only else {"dense", "masked", "masked_table", "masked_bs", "contig", "contig_bs", "small", "e5m2", "blockscaled",
                                           "channelwise", "bf16", "decode", "proj", "copy"}
    steps, warmup = args.steps, args.warmup
    extra = {}

    log("generating dense 4096^3 E4M3 inputs")
    wd = workloads.dense_square(workloads.E4M3)
    dense = None
    if "dense" in want:
        log("timing dense 4096^3 E4M3")
        dense = bench_dense(torch, f, wd, steps, warmup, timer)
        log(f"  {dense['tflops_kernel']:.1f} TFLOP/s per launch, {dense['tflops_wall']:.1f} whole-job")
    if "e5m2" in want:
        log("timing dense 4096^3 E5M2")
        w5 = workloads.dense_square(workloads.E5M2)
        r = bench_dense(torch, f, w5, steps, warmup, timer)
        extra["dense_4096_e5m2"] = {"tflops_kernel": r["tflops_kernel"], "tflops_wall": r["tflops_wall"],
                                    "kernel_ms_mean": r["kernel_ms_mean"],
                                    "frac_of_peak": r["tflops_kernel"] / PEAK_FP8_TFLOPS}
        del w5
    if "blockscaled" in want:
        log("timing block-scaled dense 4096^3 E4M3 (power-of-two scales per 1x128 / 128x128 block)")
        wbs = workloads.dense_blockscaled_square()
        r = bench_blockscaled(torch, f, wbs, steps, warmup, timer)
        extra["dense_4096_blockscaled"] = {
            "workload": "dense 4096^3 E4M3, activations N(0,1) per 1x128 block and weights N(0,0.02) per "
                        "128x128 block, each with its own power-of-two (E8M0) scale (seed 6)",
            "tflops_kernel": r["tflops_kernel"], "kernel_ms_mean": r["kernel_ms_mean"],
            "frac_of_peak": r["tflops_kernel"] / PEAK_FP8_TFLOPS}
        log(f"  {r['tflops_kernel']:.1f} TFLOP/s")
        del wbs
    if "channelwise" in want:
        log("timing dense 4096^3 E4M3 with per-row / per-channel scales and a per-channel bias")
        r = bench_channelwise(torch, f, wd, steps, warmup, timer)
        extra["dense_4096_channelwise"] = {
            "workload": "dense 4096^3 E4M3 (seed 2 operands), row scales and channel scales U[0.5,2], "
                        "bias N(0,1), applied in the epilogue",
            "tflops_kernel": r["tflops_kernel"], "kernel_ms_mean": r["kernel_ms_mean"],
            "frac_of_peak": r["tflops_kernel"] / PEAK_FP8_TFLOPS}
        log(f"  {r['tflops_kernel']:.1f} TFLOP/s")
    if "bf16" in want:
        log("timing the BF16 comparison path, 4096^3")
        wb = workloads.dense_bf16_square()
        r = bench_bf16(torch, f, wb, steps, warmup, timer)
        extra["dense_4096_bf16"] = {
            "workload": "BF16 comparison GEMM 4096^3, the seed-2 draws of the FP8 case rounded to BF16, no scales",
            "tflops_kernel": r["tflops_kernel"], "kernel_ms_mean": r["kernel_ms_mean"],
            "roofline": {"bound": "mfma", "achieved": r["tflops_kernel"], "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": r["tflops_kernel"] / PEAK_BF16_TFLOPS},
            "context_torch_matmul": {"tflops": r["torch_matmul_tflops"], "ms_mean": r["torch_matmul_ms_mean"]}}
        log(f"  {r['tflops_kernel']:.1f} TFLOP/s (torch.matmul {r['torch_matmul_tflops']:.1f})")
        del wb
    if "decode" in want:
        out = []
        for (N, K) in ((4096, 7168), (14336, 4096)):
            for M in (1, 16, 32, 64):
                r = bench_decode(torch, f, M, N, K, steps, warmup, timer)
                out.append({"M": M, "N": N, "K": K, "kernel_us_mean": r["kernel_ms_mean"] * 1e3,
                            "roofline": {"bound": "hbm", "achieved": r["gbs_kernel"], "peak": PEAK_HBM_GBS,
                                         "unit": "GB/s", "frac": r["gbs_kernel"] / PEAK_HBM_GBS,
                                         "algorithmic_bytes": r["bytes"]}})
                log(f"  decode {M}x{N}x{K}: {r['kernel_ms_mean'] * 1e3:.1f} us, {r['gbs_kernel']:.0f} GB/s")
        extra["dense_decode"] = {
            "workload": "dense few-token GEMMs, A ~N(0,1), B ~N(0,1) E4M3 (seed 13), weights rotated over "
                        "> 512 MB of copies so each launch reads them from HBM",
            "timing": "launches captured in a graph and replayed (eager calls through Python cost ~10 us each)",
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
                              "kernel_us_graph": g["kernel_ms_mean"] * 1e3}
        del a, b, o
    if "masked" in want:
        log("generating masked grouped decode inputs (G=32, cap=64, N=4096, K=7168)")
        wm = workloads.masked_decode()
        log("timing masked grouped decode")
        r = bench_masked(torch, f, wm, steps, warmup, timer)
        extra["masked_grouped"] = {
            "workload": "masked grouped FP8 GEMM, G=32, cap=64, N=4096, K=7168, m_g~U{0..32} (seed 4), E4M3, swap-AB",
            "gbs_kernel": r["gbs_kernel"], "gbs_wall": r["gbs_wall"], "kernel_ms_mean": r["kernel_ms_mean"],
            "tflops_kernel": r["tflops_kernel"], "active_experts": r["active_experts"], "valid_rows": r["valid_rows"],
            "roofline": {"bound": "hbm", "achieved": r["gbs_kernel"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": r["gbs_kernel"] / PEAK_HBM_GBS, "traffic": read_traffic("masked_decode"),
                         "algorithmic_bytes": r["bytes"]}}
        log(f"  {r['gbs_kernel']:.0f} GB/s ({r['gbs_kernel'] / PEAK_HBM_GBS:.1%} of HBM peak)")
        del wm
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
            "kernel_ms_mean": r["kernel_ms_mean"],
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
            "rows_total": r["rows_total"], "rows_valid": r["rows_valid"],
            "tflops_kernel_incl_padding": r["tflops_kernel_incl_padding"]}
        log(f"  {r['tflops_kernel']:.1f} TFLOP/s")
        del wc
    if "contig_bs" in want:
        log("generating block-scaled contiguous grouped prefill inputs")
        wcb = workloads.contig_blockscaled(8192, 8, 32, 4096, 7168, seed=9)
        r = bench_contig_blockscaled(torch, f, wcb, max(5, steps // 5), max(2, warmup // 5), timer)
        extra["contig_grouped_blockscaled"] = {
            "workload": "block-scaled contiguous grouped FP8 GEMM, 8192 tokens x top-8 over 32 experts, N=4096, "
                        "K=7168, E8M0 scales per 1x128 token block and 128x128 weight block (seed 9)",
            "tflops_kernel": r["tflops_kernel"], "kernel_ms_mean": r["kernel_ms_mean"],
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
                        "variant": f.plan(0, M, N, K).variant})
            log(f"  projection {M}x{N}x{K}: {r['tflops_kernel']:.1f} TFLOP/s")
            del wp
        extra["projections"] = out

    if "copy" in want:
        log("timing the 1 GiB copy used to calibrate the HBM byte counters")
        r = bench_copy(torch, steps, warmup, timer)
        extra["copy_1gib"] = {"gbs_kernel": r["gbs_kernel"], "kernel_ms_mean": r["kernel_ms_mean"]}
        log(f"  {r['gbs_kernel']:.0f} GB/s read+write")

    cpu = None
    if not args.no_cpu and dense is not None:
        log("timing the CPU oracle on a row sample")
        cpu = cpu_baseline(wd)

    if dense is None:
        print(json.dumps({"metric": METRIC, "partial": True, **extra}))
        return
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
                     "frac": dense["tflops_kernel"] / PEAK_FP8_TFLOPS, "traffic": read_traffic("dense_4096_e4m3"),
                     "kernel_ms_mean": dense["kernel_ms_mean"],
                     "algorithmic_flops": dense["flops"], "algorithmic_bytes": dense["bytes"]},
        "cpu_baseline": cpu,
        "kernel_source_hash": kernel_source_hash(),
    }
    line.update(extra)
    print(json.dumps(line))


if __name__ == "__main__":
    main()
