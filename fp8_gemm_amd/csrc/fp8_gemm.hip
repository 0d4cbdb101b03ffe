// C ABI of the gfx950 FP8 GEMM library: argument validation, shape-class
// dispatch (including the swap-AB choice) and kernel launch on the caller's
// stream.  See include/fp8_gemm.h for the contract of every entry point.
#include <hip/hip_runtime.h>

#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "../../include/fp8_gemm.h"
#include "kernels.hpp"

namespace {

using fp8g::GemmParams;

thread_local char g_detail[512];
thread_local char g_message[768];

int fail(int status, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_detail, sizeof g_detail, fmt, ap);
    va_end(ap);
    return status;
}

int ok() {
    g_detail[0] = '\0';
    return FP8G_OK;
}

constexpr int64_t kMaxRowStride = (int64_t(1) << 23) - 16;   // keeps 256 rows of offsets below 2^31
constexpr int kSwapMaxM = 64;                                  // swap-AB threshold of the dense form
constexpr int kSwapWideMaxM = 192;                             // masked form: one pass over the weights up to here
#ifndef SWAP_DEPTH
#define SWAP_DEPTH 2
#endif
constexpr int kSwapWaveRows = 128;                             // weight rows per wave, grouped forms
constexpr int kDecodeRows = 16;                                // weight rows per decode workgroup (one block)
constexpr int kSwapDepth = SWAP_DEPTH;                         // K blocks of loads in flight + 1
constexpr int kContigAlign = 128;                              // row alignment of experts (contiguous form)
#ifndef TILE128_WM
#define TILE128_WM 2
#define TILE128_WN 4
#endif
#ifndef T256_WM
#define T256_WM 4
#define T256_WN 2
#endif
#ifndef T256_ST
#define T256_ST 2
#define T256_BK 128
#endif
#ifndef T128_ST
#define T128_ST 3
#define T128_BK 128
#endif

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
bool dtype_ok(int d) { return d == FP8G_E4M3 || d == FP8G_E5M2; }

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ---------------------------------------------------------------------------
// Shape-class choice.
// ---------------------------------------------------------------------------
enum Variant {
    V_NONE = 0, V_TILE_256x256 = 1, V_TILE_128x256 = 2, V_SWAP = 3, V_DECODE = 4, V_TILE_256x192 = 5, V_TILE_256x224 = 6
};


// Swapped streaming kernel: 128 weight rows per wave (512 per workgroup), or
// 64 when that would leave CUs idle (16 groups of N = 4096: 128 workgroups
// of 512 rows ran at 4.4 TB/s).
int swap_wave_rows(int64_t groups, int64_t n) { return groups * cdiv(n, 4 * kSwapWaveRows) >= 256 ? kSwapWaveRows : kSwapWaveRows / 2; }

int token_blocks_for(int m) {
    if (m <= 16) return 1;
    if (m <= 32) return 2;
    if (m <= 64) return 4;
    if (m <= 128) return 8;
    return 12;
}

// Decode kernel (M <= 64): a workgroup takes 16 RB weight rows and the
// 16 CB-row token blocks, over all K or over one split of the K steps.
// Every workgroup reads all its split's token bytes, so fewer, larger row
// blocks cut the token traffic per CU: 32 rows (RB = 2) where that still
// leaves at least 256 workgroups (N = 14336: 896 workgroups of 16 rows read
// 3.5 copies of the tokens per CU, 448 of 32 rows 1.75).  When the row blocks
// are fewer than 256 (N < 4096), K is split over up to ceil(256 / blocks)
// workgroups per block (at least 4 K steps each, one per wave) so the chip
// stays full; their FP32 partial sums meet in a workspace (kSplitWs below).
//
// The waves-on-rows kernel (RB = 4: 64 weight rows per workgroup, the 4
// waves on 16 rows each, sharing one copy of the tokens per K step) is taken
// instead where it measured faster, graph-timed on one box:
//  - where the blocks above leave the CUs unevenly loaded (more than 256, not
//    a multiple of 256), at every M: N = 5120 .. 14336 (64 x 14336 x 4096:
//    19.9 -> 15.7 us, 64 x 7168 x 4096: 13.9 -> 11.3, 1 x 7168 x 4096: 8.9 ->
//    8.3, 64 x 5120 x 7168: 21.1 -> 13.9);
//  - with more than 32 tokens and at least 28 K steps per split, where the
//    token copies dominate (64 x 4096 x 14336: 21.9 -> 18.6 us, 64 x 16384 x
//    4096: 21.3 -> 17.2, 64 x 8192 x 7168: 16.8 -> 16.3).
// Its splits: as many as keep at least 16 K steps each and at most 256
// workgroups (512 with one token block); not taken below 160 workgroups or
// 16 K steps, nor with one token block over 16-row blocks beyond 64 K steps
// (1 x 7168 x 16384: 24.4 us on the waves-on-K kernel, 27.6-35.5 with 1-4
// splits; 16 x 7168 x 16384: 26.8 against 28.0; up to 64 steps it won,
// 1 x 7168 x 8192 with 4 splits 14.25 -> 13.87).
// At 64 x 4096 x 7168 (4 splits of 14 steps) it measured 13.2 against 12.4
// us, and with 32 or fewer tokens on balanced grids it was 1-7% slower.
struct DecodeShape {
    int rb, cb, blocks, splits, ksteps;
};

DecodeShape decode_shape(int64_t m, int64_t n, int64_t k) {
    DecodeShape d;
    d.cb = token_blocks_for((int)m);
    d.rb = cdiv(n, 2 * kDecodeRows) >= 256 ? 2 : 1;
    d.blocks = (int)cdiv(n, 16 * d.rb);
    const int nk = (int)cdiv(k, 128);
    d.splits = 1;
    d.ksteps = nk;
    if (d.blocks < 256 && nk >= 8) {
        int want = (int)cdiv(256, d.blocks);
        if (want > nk / 4) want = nk / 4;
        if (want > 1) {
            d.ksteps = (int)cdiv(nk, want);
            d.splits = (int)cdiv(nk, d.ksteps);   // no empty split
        }
        return d;
    }
    // waves on rows (never with fewer than 16 K steps, K = 0 included)
    if (nk < 16 || n <= 0) return d;
    const int64_t rblocks = cdiv(n, 64);
    const bool uneven = d.blocks % 256 != 0;
    int64_t want = (d.cb == 1 ? 512 : 256) / rblocks;
    if (want > nk / 16) want = nk / 16;
    if (want < 1) want = 1;
    const int64_t ksteps = cdiv(nk, want);
    const int64_t splits = cdiv(nk, ksteps);
    // one token block over 16-row blocks: the waves-on-K kernel's long loops
    // (two workgroups on most CUs) stream as fast beyond 64 K steps
    const bool short_tokens_long_k = d.cb == 1 && d.rb == 1 && nk > 64;
    if (rblocks * splits >= 160 && !short_tokens_long_k && (uneven || (d.cb == 4 && ksteps >= 28))) {
        d.rb = 4;
        d.blocks = (int)rblocks;
        d.splits = (int)splits;
        d.ksteps = (int)ksteps;
    }
    return d;
}

// Workspace of the split-K few-token path, per device: the FP32 partial sums
// of the splits (16 RB x 16 CB outputs, at most 64 x 64, per workgroup) and
// one arrival count per block of weight rows, each in its own 128-byte line.
// The waves-on-K kernel splits only with fewer than 256 blocks, so blocks x
// splits < 256 + blocks < 512 workgroups; the waves-on-rows kernel at most
// 256 blocks over 256 workgroups (512 with one token block, 4 KiB of sums
// each).  So at most 512 x 16 KiB of partial sums and 256 counts (32 KiB),
// whatever the shape.
constexpr int kSplitMaxWgs = 512;
constexpr int kSplitMaxBlocks = 256;
constexpr size_t kSplitPartialBytes = (size_t)kSplitMaxWgs * 64 * 64 * sizeof(float);
constexpr size_t kSplitCountBytes = (size_t)kSplitMaxBlocks * fp8g::kCountStride * sizeof(int);
constexpr size_t kSplitWsBytes = kSplitPartialBytes + kSplitCountBytes;

// Masked form with 65..192 tokens per group ("wide"): 8 or 12 token blocks
// in one pass over the weights, 64 weight rows per wave (the accumulators of
// 12 blocks x 8 weight blocks would not fit a wave's registers).  The weights
// stream from HBM once, as for few tokens; 128-row tiles read each group's
// weights once per 128 tokens and were measured slower at 96 and 160 tokens
// (the swap-AB benchmark table).
int swap_rows_for(int64_t groups, int64_t n, int token_blocks) {
    return token_blocks >= 8 ? kSwapWaveRows / 2 : swap_wave_rows(groups, n);
}

// Dense tiled kernel: pick the tile whose waves of 256 workgroups (one per CU)
// give the smallest estimated time.  A 128x256 tile does half the work of a
// 256x256 tile at a somewhat lower efficiency (more operand traffic per FLOP);
// 256x224 and 256x192 tiles (per-tensor and per-channel FP8 only) do seven
// eighths and three quarters of it, and win where whole waves of them replace
// a partial wave of 256x256 tiles (2048 x 14336: 512 tiles of 256x224, two
// full waves, against 448; 2048 x 12288: 512 of 256x192 against 384).
int pick_dense_tile(int64_t M, int64_t N, bool allow_narrow) {
    const int64_t t256 = cdiv(M, 256) * cdiv(N, 256);
    const int64_t t128 = cdiv(M, 128) * cdiv(N, 256);
    const int64_t t224 = cdiv(M, 256) * cdiv(N, 224);
    const int64_t t192 = cdiv(M, 256) * cdiv(N, 192);
    const double c256 = (double)cdiv(t256, 256) * 2.0;
    const double c128 = (double)cdiv(t128, 256) * 1.15;
    const double c224 = allow_narrow ? (double)cdiv(t224, 256) * 1.85 : 1e30;
    const double c192 = allow_narrow ? (double)cdiv(t192, 256) * 1.65 : 1e30;
    int best = V_TILE_256x256;
    double cost = c256;
    if (c224 < cost) best = V_TILE_256x224, cost = c224;
    if (c192 < cost) best = V_TILE_256x192, cost = c192;
    if (c128 < cost) best = V_TILE_128x256, cost = c128;
    return best;
}

void fill_decode_plan(int m, int n, int k, fp8g_plan *out) {
    const DecodeShape d = decode_shape(m, n, k);
    out->variant = V_DECODE;
    out->tile_m = 16 * d.cb;
    out->tile_n = 16 * d.rb;
    out->token_blocks = d.cb;
    out->k_splits = d.splits;
    // split K: 8 ceil(blocks / 8) x splits workgroups, so that all splits of
    // a block run on one XCD (the kernel's placement)
    out->workgroups = d.splits > 1 ? (int64_t)8 * cdiv(d.blocks, 8) * d.splits : (int64_t)d.blocks;
}

// Small problems (M <= 256 where the tiled kernel would start at most 2
// workgroups, as for 256^3): the decode kernel over 64-token tiles instead,
// one workgroup per (16 weight rows, 64 tokens), K not split.  The work is
// a few microseconds of latency either way; 64 workgroups load and store
// their parts in parallel where 2 would each carry half of the problem.
constexpr int kSmallMaxM = 256;
constexpr int kSmallMaxTiles = 2;

bool small_class(int m, int64_t tiled_workgroups) { return m > kSwapMaxM && m <= kSmallMaxM && tiled_workgroups <= kSmallMaxTiles; }

void fill_small_plan(int m, int n, fp8g_plan *out) {
    out->variant = V_DECODE;
    out->tile_m = 64;
    out->tile_n = 16;
    out->token_blocks = 4;
    out->k_splits = 1;
    out->workgroups = cdiv(n, 16) * cdiv(m, 64);
}

int tile_m_of(int variant) { return variant == V_TILE_128x256 ? 128 : 256; }
int tile_n_of(int variant) { return variant == V_TILE_256x192 ? 192 : variant == V_TILE_256x224 ? 224 : 256; }

int plan_impl(int op, int m, int n, int k, int groups, int expected_m, fp8g_plan *out) {
    memset(out, 0, sizeof *out);
    out->k_splits = 1;
    if (m < 0 || n < 0 || k < 0 || groups < 0) return fail(FP8G_ERR_SHAPE, "negative size (m=%d n=%d k=%d groups=%d)", m, n, k, groups);
    // K in bytes: 16-byte chunks of the ring (BF16: 2 bytes per element)
    const int64_t kbytes = op == 4 ? 2 * (int64_t)k : k;
    if (kbytes % 16 != 0) return fail(FP8G_ERR_SHAPE, "K=%d is not a multiple of %d", k, op == 4 ? 8 : 16);
    if (kbytes > kMaxRowStride) return fail(FP8G_ERR_SHAPE, "K=%d exceeds the row-stride limit %lld bytes", k, (long long)kMaxRowStride);
    if (op == 0) {
        if (m == 0 || n == 0) return ok();
        if (m <= kSwapMaxM) {
            fill_decode_plan(m, n, k, out);
        } else {
            out->variant = pick_dense_tile(m, n, true);
            out->tile_m = tile_m_of(out->variant);
            out->tile_n = tile_n_of(out->variant);
            out->workgroups = cdiv(m, out->tile_m) * cdiv(n, out->tile_n);
            if (small_class(m, out->workgroups)) fill_small_plan(m, n, out);
        }
        return ok();
    }
    if (op == 1) {
        if (expected_m < 0 || expected_m > m)
            return fail(FP8G_ERR_ARG, "expected_m=%d outside [0, cap=%d]", expected_m, m);
        if (groups == 0 || m == 0 || n == 0) return ok();
        const int hint = expected_m > 0 ? expected_m : m;
        if (hint <= kSwapWideMaxM) {
            out->variant = V_SWAP;
            out->token_blocks = token_blocks_for(hint);
            out->tile_m = 16 * out->token_blocks;
            out->tile_n = 4 * swap_rows_for(groups, n, out->token_blocks);
            out->workgroups = (int64_t)groups * cdiv(n, out->tile_n);
        } else {
            out->variant = V_TILE_128x256;
            out->tile_m = 128;
            out->tile_n = 256;
            out->workgroups = (int64_t)groups * cdiv(m, 128) * cdiv(n, 256);
        }
        return ok();
    }
    if (op == 2 || op == 5) {
        if (m == 0 || n == 0) return ok();
        if (groups == 0) return fail(FP8G_ERR_SHAPE, "G=0 with M_total=%d rows", m);
        out->variant = V_TILE_256x256;
        out->tile_m = 2 * kContigAlign;
        out->tile_n = 256;
        if (op == 2)
            // 256-row tiles on the 8-wave kernel, then one workgroup per tile
            // for its second 128-row block, which computes only when that
            // block's expert differs
            out->workgroups = 2 * cdiv(m, 2 * kContigAlign) * cdiv(n, 256);
        else
            // block scales: run-aligned 256-row tiles (128 rows at the end of
            // a run with an odd number of 128-row blocks) on the 4-wave
            // kernel; one workgroup per slot of two blocks computes the tiles
            // that start in it
            out->workgroups = cdiv(cdiv(m, kContigAlign), 2) * cdiv(n, 256);
        return ok();
    }
    if (op == 3) {
        // Block-scaled dense: the decode kernel for few tokens, else the tiled
        // kernel (block scales applied per 128-byte K step of its ring).
        if (m == 0 || n == 0) return ok();
        if (m <= kSwapMaxM) {
            fill_decode_plan(m, n, k, out);
            return ok();
        }
        out->variant = pick_dense_tile(m, n, false);
        out->tile_m = tile_m_of(out->variant);
        out->tile_n = 256;
        out->workgroups = cdiv(m, out->tile_m) * cdiv(n, 256);
        if (small_class(m, out->workgroups)) fill_small_plan(m, n, out);
        return ok();
    }
    if (op == 4) {
        // BF16 comparison path: always the tiled kernel.
        if (m == 0 || n == 0) return ok();
        out->variant = pick_dense_tile(m, n, false);
        out->tile_m = tile_m_of(out->variant);
        out->tile_n = 256;
        out->workgroups = cdiv(m, out->tile_m) * cdiv(n, 256);
        return ok();
    }
    return fail(FP8G_ERR_ARG, "unknown op %d", op);
}

// ---------------------------------------------------------------------------
// Device check: the code objects are built for gfx950 only.
// ---------------------------------------------------------------------------
int check_device() {
    static int cached[64];   // 0 unknown, 1 ok, -1 unsupported
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(FP8G_ERR_UNSUPPORTED, "no HIP device");
    if (dev >= 0 && dev < 64 && cached[dev] == 1) return FP8G_OK;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return fail(FP8G_ERR_UNSUPPORTED, "cannot query device %d", dev);
    const bool good = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    if (dev >= 0 && dev < 64) cached[dev] = good ? 1 : -1;
    if (!good) return fail(FP8G_ERR_UNSUPPORTED, "device %d is %s; this library is built for gfx950 only", dev, prop.gcnArchName);
    return FP8G_OK;
}

int launch_status(const char *what) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(FP8G_ERR_LAUNCH, "%s launch failed: %s", what, hipGetErrorString(e));
    return ok();
}

// ---------------------------------------------------------------------------
// Launch helpers: one instantiation per (operand formats, tile shape, mode).
// ---------------------------------------------------------------------------
// BF16: the BF16 instantiation only (dense, no scales); otherwise the four
// FP8 format pairs.
template <int BM, int BN, int WM, int WN, int STAGES, int BK, int MODE, int SCL = 0, bool BF16 = false>
int launch_ring(int fa, int fb, const GemmParams &p, dim3 grid, hipStream_t s) {
    const dim3 block(64 * WM * WN);
#define FP8G_RING(FA, FB) \
    hipLaunchKernelGGL((fp8g::ring_kernel<BM, BN, WM, WN, FA, FB, MODE, STAGES, BK, SCL>), grid, block, 0, s, p)
    if constexpr (BF16) {
        static_assert(MODE == fp8g::MODE_DENSE && SCL == fp8g::SCALE_TENSOR, "BF16: dense, no scales");
        FP8G_RING(fp8g::FMT_BF16, fp8g::FMT_BF16);
        return launch_status("tiled kernel (BF16)");
    } else {
        if (fa == 0 && fb == 0) FP8G_RING(0, 0);
        else if (fa == 0 && fb == 1) FP8G_RING(0, 1);
        else if (fa == 1 && fb == 0) FP8G_RING(1, 0);
        else FP8G_RING(1, 1);
        return launch_status("tiled kernel");
    }
#undef FP8G_RING
}

template <int BM, int STAGES, int MODE, int SCL, int BN = 256>
int launch_tile16(int fa, int fb, const GemmParams &p, dim3 grid, hipStream_t s) {
    const dim3 block(256);
    // K not a multiple of 128: the variant with the per-lane check of the last step
#define FP8G_T16(FA, FB)                                                                                     \
    do {                                                                                                      \
        if (p.K % 128)                                                                                        \
            hipLaunchKernelGGL((fp8g::tile16_kernel<BM, BN, STAGES, FA, FB, MODE, SCL, true>), grid, block, 0, s, p); \
        else                                                                                                  \
            hipLaunchKernelGGL((fp8g::tile16_kernel<BM, BN, STAGES, FA, FB, MODE, SCL, false>), grid, block, 0, s, p); \
    } while (0)
    if (fa == 0 && fb == 0) FP8G_T16(0, 0);
    else if (fa == 0 && fb == 1) FP8G_T16(0, 1);
    else if (fa == 1 && fb == 0) FP8G_T16(1, 0);
    else FP8G_T16(1, 1);
#undef FP8G_T16
    return launch_status("tiled kernel (16x16x128)");
}

// Tile shapes of the tiled kernels: 256 x 256 and 128 x 256 (and, below, 256 x
// 224 and 256 x 192 for dense FP8 without block scales).  FP8 (dense forms and
// the contiguous grouped form) runs on 4 waves and the 16x16x128 instruction
// (2-slot ring, 128 KB of LDS, for 256 rows; 3-slot, 144 KB, for 128 rows);
// BF16 and the masked grouped form's tiles on 8 waves and 32x32x64 (4 x 2
// waves and a 2-slot ring for 256 rows, 2 x 4 and 3 slots for 128).
template <int MODE, int SCL = 0>
int launch_tile256(int fa, int fb, const GemmParams &p, dim3 grid, hipStream_t s) {
    static_assert(MODE == fp8g::MODE_DENSE, "256-row tiles of the dense forms");
    if (fa != fp8g::FMT_BF16) return launch_tile16<256, 2, MODE, SCL>(fa, fb, p, grid, s);
    if constexpr (SCL == fp8g::SCALE_TENSOR)
        return launch_ring<256, 256, T256_WM, T256_WN, T256_ST, T256_BK, MODE, SCL, true>(fa, fb, p, grid, s);
    else
        return fail(FP8G_ERR_ARG, "BF16 operands take no scales");
}
// 256 x 224 and 256 x 192 tiles: dense FP8 with per-tensor or per-channel scales.
template <int SCL>
int launch_tile256_narrow(int variant, int fa, int fb, const GemmParams &p, dim3 grid, hipStream_t s) {
    static_assert(SCL != fp8g::SCALE_BLOCK, "block scales: 256-column tiles");
    if (variant == V_TILE_256x224) return launch_tile16<256, 2, fp8g::MODE_DENSE, SCL, 224>(fa, fb, p, grid, s);
    return launch_tile16<256, 2, fp8g::MODE_DENSE, SCL, 192>(fa, fb, p, grid, s);
}
template <int MODE, int SCL = 0>
int launch_tile128(int fa, int fb, const GemmParams &p, dim3 grid, hipStream_t s) {
    if constexpr (MODE == fp8g::MODE_DENSE) {
        if (fa != fp8g::FMT_BF16) return launch_tile16<128, 3, MODE, SCL>(fa, fb, p, grid, s);
        if constexpr (SCL == fp8g::SCALE_TENSOR)
            return launch_ring<128, 256, TILE128_WM, TILE128_WN, T128_ST, T128_BK, MODE, SCL, true>(fa, fb, p, grid, s);
        else
            return fail(FP8G_ERR_ARG, "BF16 operands take no scales");
    } else {
        return launch_ring<128, 256, TILE128_WM, TILE128_WN, T128_ST, T128_BK, MODE, SCL>(fa, fb, p, grid, s);
    }
}

template <int WR, int CB, int MODE, int SCL = 0>
int launch_swap_cb(int fa, int fb, const GemmParams &p, dim3 grid, hipStream_t s) {
    const dim3 block(256);
#define FP8G_SWAP(FA, FB) \
    hipLaunchKernelGGL((fp8g::swap_kernel<WR, CB, FA, FB, kSwapDepth, MODE, SCL>), grid, block, 0, s, p)
    if (fa == 0 && fb == 0) FP8G_SWAP(0, 0);
    else if (fa == 0 && fb == 1) FP8G_SWAP(0, 1);
    else if (fa == 1 && fb == 0) FP8G_SWAP(1, 0);
    else FP8G_SWAP(1, 1);
#undef FP8G_SWAP
    return launch_status("swap kernel");
}

template <int WR, int MODE, int SCL>
int launch_swap_wr(int cb, int fa, int fb, const GemmParams &p, dim3 grid, hipStream_t s) {
    if (cb == 1) return launch_swap_cb<WR, 1, MODE, SCL>(fa, fb, p, grid, s);
    if (cb == 2) return launch_swap_cb<WR, 2, MODE, SCL>(fa, fb, p, grid, s);
    return launch_swap_cb<WR, 4, MODE, SCL>(fa, fb, p, grid, s);
}

// p.tiles_n must hold the number of plan.tile_n-row weight blocks of a group.
template <int MODE, int SCL = 0>
int launch_swap(const fp8g_plan &plan, int fa, int fb, const GemmParams &p, hipStream_t s) {
    const dim3 grid((unsigned)plan.workgroups);
    if (plan.token_blocks == 8) return launch_swap_cb<kSwapWaveRows / 2, 8, MODE, SCL>(fa, fb, p, grid, s);
    if (plan.token_blocks == 12) return launch_swap_cb<kSwapWaveRows / 2, 12, MODE, SCL>(fa, fb, p, grid, s);
    if (plan.tile_n == 4 * kSwapWaveRows) return launch_swap_wr<kSwapWaveRows, MODE, SCL>(plan.token_blocks, fa, fb, p, grid, s);
    return launch_swap_wr<kSwapWaveRows / 2, MODE, SCL>(plan.token_blocks, fa, fb, p, grid, s);
}

// Decode kernel: 4 waves per workgroup and per-wave LDS rings, as deep as fits
// in 80 KB so that two workgroups share a CU: 5, 3 or 2 steps for 1, 2 or 4
// token blocks with one weight block, 3, 2, 2 with two (the last needs 96 KB:
// one workgroup per CU).  Measured best against 8 waves and against deeper
// rings with one workgroup per CU: rings of 8, 6 and 4 steps (160 KB) where
// the grid is at most one workgroup per CU took 7.97 / 12.97 us at M = 1 / 64,
// N = 4096, K = 7168, against 7.39 / 12.34 us with these.  Block scales add
// 512 bytes per slot.
constexpr int kDecodeWaves = 4;

// The split-K workspace of each device, allocated (and its counts zeroed) by
// the first call on that device that splits K; the kernels leave the counts
// at zero again.  Calls that split K and overlap on one device share it.
struct SplitWs {
    float *partial = nullptr;
    int *count = nullptr;
};
std::mutex g_ws_mutex;
SplitWs g_ws[64];

// The device's workspace in `ws`, or none (ws.partial == NULL: the caller does
// not split K) when it does not exist yet and `stream` is being captured into
// a graph, where no allocation may happen.
int split_workspace(hipStream_t stream, SplitWs &ws) {
    ws = SplitWs{};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return fail(FP8G_ERR_UNSUPPORTED, "no usable HIP device");
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    if (!g_ws[dev].partial) {
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        if (hipStreamIsCapturing(stream, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) return ok();
        void *mem = nullptr;
        if (hipMalloc(&mem, kSplitWsBytes) != hipSuccess)
            return fail(FP8G_ERR_LAUNCH, "cannot allocate the %zu-byte split-K workspace", kSplitWsBytes);
        int *count = reinterpret_cast<int *>(static_cast<char *>(mem) + kSplitPartialBytes);
        if (hipMemsetAsync(count, 0, kSplitCountBytes, stream) != hipSuccess) {
            (void)hipFree(mem);
            return fail(FP8G_ERR_LAUNCH, "cannot clear the split-K workspace");
        }
        g_ws[dev].partial = static_cast<float *>(mem);
        g_ws[dev].count = count;
    }
    ws = g_ws[dev];
    return ok();
}

// Grids of at most 256 workgroups take the one-per-CU build, with 16 KB of
// dynamic LDS that takes every instance past 80 KB, so that no CU holds two
// of them while another holds none; larger grids take the two-per-CU build
// (N = 7168, 448 workgroups: 10.07 -> 9.38 us at M = 1, K = 4096).
constexpr unsigned kDecodeSpreadPad = 16 * 1024;

// Steps of token copies in flight in the waves-on-rows decode kernel (the
// weights run one step further ahead).  2 measured up to 13% faster than 1
// (64 x 14336 x 4096: 18.0 -> 15.7 us; 64 x 4096 x 7168 with 4 splits: 14.4
// -> 13.2).  Without a K split 3 is 1-2% faster still (32 x 14336 x 4096:
// 14.71 -> 14.43 us, 64 x 12288 x 4096: 14.76 -> 14.53); with splits 3 was
// even with 2 or slower (1 x 14336 x 4096, 2 splits: 13.44 -> 13.69).
constexpr int kDecodeRowsLead = 2;
constexpr int kDecodeRowsLeadUnsplit = 3;

// Ring slots per wave of the waves-on-K decode kernel: 3 with one token
// block over 16-row blocks, else 2.  Deeper rings measured slower, shallower
// ones faster, interleaved on one box (1 x 4096 x 7168: 7.48 us with 5 slots,
// 7.31 with 3; 16 x 4096 x 7168 8.16 -> 7.97; 1 x 4096 x 4096 6.22 -> 5.95;
// 32 x 4096 x 7168 with 2 instead of 3 slots 9.69 -> 9.54; 16 x 8192 x 7168
// with 2 instead of 3, 12.21 -> 11.92): with one step of weights already in
// flight per wave across 4 waves, more slots only delay the first step.
template <int RB, int CB, int SCL>
int launch_decode_cb(int fa, int fb, const GemmParams &p, dim3 grid, hipStream_t s) {
    constexpr int D = RB == 1 && CB == 1 ? 3 : 2;
    const dim3 block(64 * kDecodeWaves);
    const bool one = (int64_t)grid.x * grid.y <= 256;
#define FP8G_DEC(FA, FB)                                                                                   \
    do {                                                                                                    \
        if (one)                                                                                            \
            hipLaunchKernelGGL((fp8g::decode_kernel<kDecodeWaves, RB, CB, FA, FB, D, SCL, 1>), grid, block, \
                               kDecodeSpreadPad, s, p);                                                     \
        else                                                                                                \
            hipLaunchKernelGGL((fp8g::decode_kernel<kDecodeWaves, RB, CB, FA, FB, D, SCL, 2>), grid, block, 0, s, p); \
    } while (0)
    if (fa == 0 && fb == 0) FP8G_DEC(0, 0);
    else if (fa == 0 && fb == 1) FP8G_DEC(0, 1);
    else if (fa == 1 && fb == 0) FP8G_DEC(1, 0);
    else FP8G_DEC(1, 1);
#undef FP8G_DEC
    return launch_status("decode kernel");
}

template <int RB, int SCL>
int launch_decode_rb(int cb, int fa, int fb, const GemmParams &p, dim3 grid, hipStream_t s) {
    if (cb == 1) return launch_decode_cb<RB, 1, SCL>(fa, fb, p, grid, s);
    if (cb == 2) return launch_decode_cb<RB, 2, SCL>(fa, fb, p, grid, s);
    return launch_decode_cb<RB, 4, SCL>(fa, fb, p, grid, s);
}

// The waves-on-rows decode kernel (64 weight rows per workgroup).  Grids of
// at most 256 workgroups are spread one per CU, as above: dynamic LDS takes
// every instance past half of the CU's 160 KB.
template <int CB, int SCL, int LT>
int launch_decode_rows_lt(int fa, int fb, const GemmParams &p, dim3 grid, hipStream_t s) {
    constexpr int smem = fp8g::RowsDecodeLayout<CB, SCL, LT>::SMEM;
    const unsigned pad = (int64_t)grid.x * grid.y <= 256 && smem <= 80 * 1024 ? (unsigned)(80 * 1024 + 1024 - smem) : 0u;
    const dim3 block(256);
#define FP8G_DROWS(FA, FB) hipLaunchKernelGGL((fp8g::decode_rows_kernel<CB, FA, FB, SCL, LT, 1>), grid, block, pad, s, p)
    if (fa == 0 && fb == 0) FP8G_DROWS(0, 0);
    else if (fa == 0 && fb == 1) FP8G_DROWS(0, 1);
    else if (fa == 1 && fb == 0) FP8G_DROWS(1, 0);
    else FP8G_DROWS(1, 1);
#undef FP8G_DROWS
    return launch_status("decode kernel (waves on rows)");
}

template <int SCL, int LT>
int launch_decode_rows_cb(int cb, int fa, int fb, const GemmParams &p, dim3 grid, hipStream_t s) {
    if (cb == 1) return launch_decode_rows_lt<1, SCL, LT>(fa, fb, p, grid, s);
    if (cb == 2) return launch_decode_rows_lt<2, SCL, LT>(fa, fb, p, grid, s);
    return launch_decode_rows_lt<4, SCL, LT>(fa, fb, p, grid, s);
}

template <int SCL>
int launch_decode_rows(int cb, int fa, int fb, const GemmParams &p, dim3 grid, hipStream_t s) {
    if (p.splits > 1) return launch_decode_rows_cb<SCL, kDecodeRowsLead>(cb, fa, fb, p, grid, s);
    return launch_decode_rows_cb<SCL, kDecodeRowsLeadUnsplit>(cb, fa, fb, p, grid, s);
}

// K split as the plan says when `ws` holds a workspace, else over the 4 waves
// only (waves on K), or not at all (waves on rows).
template <int SCL>
int launch_decode(const fp8g_plan &plan, int fa, int fb, GemmParams p, const SplitWs &ws, hipStream_t s) {
    const int rb = plan.tile_n / 16, cb = plan.token_blocks;
    // x: one workgroup per block of weight rows; y: the 64-token tiles (all M
    // at once for M <= 64), or (split K, M <= 64) the splits, x then padded
    // to a multiple of 8 so that all splits of a block run on one XCD
    const unsigned mtiles = p.M > kSwapMaxM ? (unsigned)cdiv(p.M, 64) : 1u;
    dim3 grid((unsigned)cdiv(p.N, 16 * rb), mtiles);
    p.splits = 1;
    if (plan.k_splits > 1 && ws.partial) {
        p.splits = plan.k_splits;
        p.ksteps = (int)cdiv(cdiv(p.K, 128), plan.k_splits);
        p.ws = ws.partial;
        p.cnt = ws.count;
        grid = dim3((unsigned)(8 * cdiv(grid.x, 8)), (unsigned)plan.k_splits);
    }
    if (rb == 4) return launch_decode_rows<SCL>(cb, fa, fb, p, grid, s);
    if (rb == 2) return launch_decode_rb<2, SCL>(cb, fa, fb, p, grid, s);
    return launch_decode_rb<1, SCL>(cb, fa, fb, p, grid, s);
}

// The workspace a decode plan needs (none unless it splits K).
int decode_workspace(const fp8g_plan &plan, hipStream_t s, SplitWs &ws) {
    ws = SplitWs{};
    if (plan.variant != V_DECODE || plan.k_splits <= 1) return ok();
    return split_workspace(s, ws);
}

__global__ void clear_counts(int *count, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) count[fp8g::kCountStride * i] = 0;
}

}  // namespace

// Scratch of the allocation-free entry point (fp8_gemm_nt_noalloc): the
// split-K workspace's layout and bound (kSplitWsBytes: 8 MiB of partial sums
// and 256 counts) in a device array of this library's code object.  Each
// device holds its own copy, from the library's load until the process ends.
// In host code `scratch` only names the symbol; its device address comes from
// hipGetSymbolAddress (scratch_workspace below).
static __device__ __align__(256) unsigned char scratch[kSplitWsBytes];

namespace {

std::mutex g_scratch_mutex;
SplitWs g_scratch[64];

// The scratch array of the current device as a split-K workspace.  The first
// call on a device looks up the array's address there (and keeps it) and
// clears its counts with a small kernel on `stream` (no memset: the call may
// be captured into a graph); no memory is allocated.
int scratch_workspace(hipStream_t stream, SplitWs &ws) {
    ws = SplitWs{};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return fail(FP8G_ERR_UNSUPPORTED, "no usable HIP device");
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch[dev].partial) {
        void *ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr)
            return fail(FP8G_ERR_LAUNCH, "no address for the scratch array on device %d: %s", dev, hipGetErrorString(e));
        int *count = reinterpret_cast<int *>(static_cast<char *>(ptr) + kSplitPartialBytes);
        hipLaunchKernelGGL(clear_counts, dim3(1), dim3(kSplitMaxBlocks), 0, stream, count, kSplitMaxBlocks);
        const hipError_t le = hipGetLastError();
        if (le != hipSuccess) return fail(FP8G_ERR_LAUNCH, "clearing the scratch counts failed: %s", hipGetErrorString(le));
        g_scratch[dev].partial = static_cast<float *>(ptr);
        g_scratch[dev].count = count;
    }
    ws = g_scratch[dev];
    return ok();
}

// The scratch a decode plan needs, from the scratch array; sizes beyond the
// array are refused (none arise: see kSplitWsBytes).
int decode_scratch(const fp8g_plan &plan, hipStream_t s, SplitWs &ws) {
    ws = SplitWs{};
    if (plan.variant != V_DECODE || plan.k_splits <= 1) return ok();
    const int64_t blocks = plan.workgroups / plan.k_splits;
    const int64_t need = plan.workgroups * (int64_t)(plan.tile_n / 16) * plan.token_blocks * 64 * 16;
    if (blocks > kSplitMaxBlocks || need > (int64_t)kSplitPartialBytes)
        return fail(FP8G_ERR_ARG, "the split-K sums need %lld bytes and %lld counts, above the scratch maximum "
                    "of %zu bytes and %d counts", (long long)need, (long long)blocks, kSplitPartialBytes, kSplitMaxBlocks);
    return scratch_workspace(s, ws);
}

}  // namespace

extern "C" {

int fp8_gemm_abi_version(void) { return FP8G_ABI_VERSION; }

const char *fp8_gemm_strerror(int status) {
    const char *base;
    switch (status) {
        case FP8G_OK: base = "ok"; break;
        case FP8G_ERR_NULL: base = "null pointer"; break;
        case FP8G_ERR_SHAPE: base = "invalid shape"; break;
        case FP8G_ERR_ALIGN: base = "misaligned pointer or stride"; break;
        case FP8G_ERR_DTYPE: base = "invalid FP8 dtype"; break;
        case FP8G_ERR_STRIDE: base = "invalid row stride"; break;
        case FP8G_ERR_LAUNCH: base = "kernel launch failed"; break;
        case FP8G_ERR_UNSUPPORTED: base = "unsupported device"; break;
        case FP8G_ERR_ARG: base = "invalid argument"; break;
        default: base = "unknown status"; break;
    }
    if (g_detail[0]) snprintf(g_message, sizeof g_message, "%s: %s", base, g_detail);
    else snprintf(g_message, sizeof g_message, "%s", base);
    return g_message;
}

int fp8_gemm_plan(int op, int m, int n, int k, int groups, int expected_m, fp8g_plan *out) {
    if (!out) return fail(FP8G_ERR_NULL, "plan output pointer is NULL");
    return plan_impl(op, m, n, k, groups, expected_m, out);
}

}  // extern "C"

namespace {

// fp8_gemm_nt and fp8_gemm_nt_noalloc: the same kernels; the split-K decode
// path's workspace is the library-allocated one or the scratch array.
int gemm_nt_impl(const void *A, int64_t lda, int a_dtype, const void *B, int64_t ldb, int b_dtype,
                 const float *scale_a, const float *scale_b, void *D, int64_t ldd, int M, int N, int K,
                 void *stream, bool no_alloc) {
    if (!dtype_ok(a_dtype) || !dtype_ok(b_dtype)) return fail(FP8G_ERR_DTYPE, "dtypes %d, %d", a_dtype, b_dtype);
    fp8g_plan plan;
    int st = plan_impl(0, M, N, K, 1, 0, &plan);
    if (st != FP8G_OK) return st;
    if (plan.variant == V_NONE) return ok();
    if ((K > 0 && (!A || !B)) || !D || !scale_a || !scale_b)
        return fail(FP8G_ERR_NULL, "A, B (unless K = 0), D, scale_a and scale_b are required");
    if (!aligned16(A) || !aligned16(B) || !aligned16(D)) return fail(FP8G_ERR_ALIGN, "A, B and D must be 16-byte aligned");
    if (!aligned4(scale_a) || !aligned4(scale_b)) return fail(FP8G_ERR_ALIGN, "scales must be 4-byte aligned");
    if (lda < K || ldb < K) return fail(FP8G_ERR_STRIDE, "lda=%lld / ldb=%lld below K=%d", (long long)lda, (long long)ldb, K);
    if (lda % 16 || ldb % 16) return fail(FP8G_ERR_ALIGN, "lda=%lld / ldb=%lld not multiples of 16 bytes", (long long)lda, (long long)ldb);
    if (lda > kMaxRowStride || ldb > kMaxRowStride) return fail(FP8G_ERR_STRIDE, "row stride above %lld bytes", (long long)kMaxRowStride);
    if (ldd < N) return fail(FP8G_ERR_STRIDE, "ldd=%lld below N=%d", (long long)ldd, N);
    if (ldd % 8) return fail(FP8G_ERR_ALIGN, "ldd=%lld not a multiple of 8 elements", (long long)ldd);
    if ((st = check_device()) != FP8G_OK) return st;

    GemmParams p = {};
    p.A = static_cast<const uint8_t *>(A);
    p.B = static_cast<const uint8_t *>(B);
    p.D = static_cast<uint16_t *>(D);
    p.lda = lda; p.ldb = ldb; p.ldd = ldd;
    p.M = M; p.N = N; p.K = K; p.G = 1; p.cap = M;
    p.scale_a = scale_a; p.scale_b = scale_b;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int fa = a_dtype, fb = b_dtype;
    if (plan.variant == V_DECODE) {
        SplitWs ws;
        st = no_alloc ? decode_scratch(plan, s, ws) : decode_workspace(plan, s, ws);
        if (st != FP8G_OK) return st;
        return launch_decode<fp8g::SCALE_TENSOR>(plan, fa, fb, p, ws, s);
    }
    p.tiles_m = (int)cdiv(M, plan.tile_m);
    p.tiles_n = (int)cdiv(N, plan.tile_n);
    const dim3 grid((unsigned)plan.workgroups);
    if (plan.variant == V_TILE_256x256) return launch_tile256<fp8g::MODE_DENSE>(fa, fb, p, grid, s);
    if (plan.variant == V_TILE_256x192 || plan.variant == V_TILE_256x224)
        return launch_tile256_narrow<fp8g::SCALE_TENSOR>(plan.variant, fa, fb, p, grid, s);
    return launch_tile128<fp8g::MODE_DENSE>(fa, fb, p, grid, s);
}

}  // namespace

extern "C" {

int fp8_gemm_nt(const void *A, int64_t lda, int a_dtype, const void *B, int64_t ldb, int b_dtype,
                const float *scale_a, const float *scale_b, void *D, int64_t ldd, int M, int N, int K,
                void *stream) {
    return gemm_nt_impl(A, lda, a_dtype, B, ldb, b_dtype, scale_a, scale_b, D, ldd, M, N, K, stream, false);
}

int fp8_gemm_nt_noalloc(const void *A, int64_t lda, int a_dtype, const void *B, int64_t ldb, int b_dtype,
                        const float *scale_a, const float *scale_b, void *D, int64_t ldd, int M, int N, int K,
                        void *stream) {
    return gemm_nt_impl(A, lda, a_dtype, B, ldb, b_dtype, scale_a, scale_b, D, ldd, M, N, K, stream, true);
}

int bf16_gemm_nt(const void *A, int64_t lda, const void *B, int64_t ldb, void *D, int64_t ldd, int M, int N, int K,
                 void *stream) {
    fp8g_plan plan;
    int st = plan_impl(4, M, N, K, 1, 0, &plan);
    if (st != FP8G_OK) return st;
    if (plan.variant == V_NONE) return ok();
    if ((K > 0 && (!A || !B)) || !D) return fail(FP8G_ERR_NULL, "A, B (unless K = 0) and D are required");
    if (!aligned16(A) || !aligned16(B) || !aligned16(D)) return fail(FP8G_ERR_ALIGN, "A, B and D must be 16-byte aligned");
    if (lda < K || ldb < K) return fail(FP8G_ERR_STRIDE, "lda=%lld / ldb=%lld below K=%d", (long long)lda, (long long)ldb, K);
    if (lda % 8 || ldb % 8) return fail(FP8G_ERR_ALIGN, "lda=%lld / ldb=%lld not multiples of 8 elements", (long long)lda, (long long)ldb);
    if (2 * lda > kMaxRowStride || 2 * ldb > kMaxRowStride)
        return fail(FP8G_ERR_STRIDE, "row stride above %lld bytes", (long long)kMaxRowStride);
    if (ldd < N) return fail(FP8G_ERR_STRIDE, "ldd=%lld below N=%d", (long long)ldd, N);
    if (ldd % 8) return fail(FP8G_ERR_ALIGN, "ldd=%lld not a multiple of 8 elements", (long long)ldd);
    if ((st = check_device()) != FP8G_OK) return st;

    // The tiled kernel counts K and the operand strides in bytes.
    GemmParams p = {};
    p.A = static_cast<const uint8_t *>(A);
    p.B = static_cast<const uint8_t *>(B);
    p.D = static_cast<uint16_t *>(D);
    p.lda = 2 * lda; p.ldb = 2 * ldb; p.ldd = ldd;
    p.M = M; p.N = N; p.K = 2 * K; p.G = 1; p.cap = M;
    p.tiles_m = (int)cdiv(M, plan.tile_m);
    p.tiles_n = (int)cdiv(N, plan.tile_n);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const dim3 grid((unsigned)plan.workgroups);
    if (plan.variant == V_TILE_256x256)
        return launch_tile256<fp8g::MODE_DENSE>(fp8g::FMT_BF16, fp8g::FMT_BF16, p, grid, s);
    return launch_tile128<fp8g::MODE_DENSE>(fp8g::FMT_BF16, fp8g::FMT_BF16, p, grid, s);
}

int fp8_grouped_gemm_masked(const void *A, int a_dtype, const void *B, int b_dtype, const float *scale_a,
                            const float *scale_b, const int32_t *masked_m, void *D, int G, int cap, int N, int K,
                            int expected_m, void *stream) {
    if (!dtype_ok(a_dtype) || !dtype_ok(b_dtype)) return fail(FP8G_ERR_DTYPE, "dtypes %d, %d", a_dtype, b_dtype);
    if (G < 0 || cap < 0) return fail(FP8G_ERR_SHAPE, "negative G=%d or cap=%d", G, cap);
    fp8g_plan plan;
    int st = plan_impl(1, cap, N, K, G, expected_m, &plan);
    if (st != FP8G_OK) return st;
    if (plan.variant == V_NONE) return ok();
    if ((K > 0 && (!A || !B)) || !D || !scale_a || !scale_b || !masked_m)
        return fail(FP8G_ERR_NULL, "A, B (unless K = 0), D, scale_a, scale_b and masked_m are required");
    if (!aligned16(A) || !aligned16(B) || !aligned16(D)) return fail(FP8G_ERR_ALIGN, "A, B and D must be 16-byte aligned");
    if (!aligned4(scale_a) || !aligned4(scale_b) || !aligned4(masked_m)) return fail(FP8G_ERR_ALIGN, "scales and masked_m must be 4-byte aligned");
    if (N % 8) return fail(FP8G_ERR_ALIGN, "N=%d: rows of D must stay 16-byte aligned (N %% 8 == 0)", N);
    if ((st = check_device()) != FP8G_OK) return st;

    GemmParams p = {};
    p.A = static_cast<const uint8_t *>(A);
    p.B = static_cast<const uint8_t *>(B);
    p.D = static_cast<uint16_t *>(D);
    p.lda = K; p.ldb = K; p.ldd = N;
    p.a_gstride = (int64_t)cap * K;
    p.b_gstride = (int64_t)N * K;
    p.d_gstride = (int64_t)cap * N;
    p.M = cap; p.N = N; p.K = K; p.G = G; p.cap = cap;
    p.scale_a = scale_a; p.scale_b = scale_b; p.masked_m = masked_m;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (plan.variant == V_SWAP) {
        p.tiles_m = 1;
        p.tiles_n = (int)cdiv(N, plan.tile_n);
        return launch_swap<fp8g::MODE_MASKED>(plan, a_dtype, b_dtype, p, s);
    }
    p.tiles_m = (int)cdiv(cap, 128);
    p.tiles_n = (int)cdiv(N, 256);
    return launch_tile128<fp8g::MODE_MASKED>(a_dtype, b_dtype, p, dim3((unsigned)(p.tiles_m * p.tiles_n), (unsigned)G), s);
}

int fp8_grouped_gemm_masked_blockscaled(const void *A, int a_dtype, const void *B, int b_dtype,
                                        const uint8_t *scale_a, int64_t lds_a, const uint8_t *scale_b, int64_t lds_b,
                                        const int32_t *masked_m, void *D, int G, int cap, int N, int K,
                                        int expected_m, void *stream) {
    if (!dtype_ok(a_dtype) || !dtype_ok(b_dtype)) return fail(FP8G_ERR_DTYPE, "dtypes %d, %d", a_dtype, b_dtype);
    if (G < 0 || cap < 0) return fail(FP8G_ERR_SHAPE, "negative G=%d or cap=%d", G, cap);
    fp8g_plan plan;
    int st = plan_impl(1, cap, N, K, G, expected_m, &plan);
    if (st != FP8G_OK) return st;
    if (plan.variant == V_NONE) return ok();
    if ((K > 0 && (!A || !B || !scale_a || !scale_b)) || !D || !masked_m)
        return fail(FP8G_ERR_NULL, "A, B, scale_a, scale_b (unless K = 0), D and masked_m are required");
    if (!aligned16(A) || !aligned16(B) || !aligned16(D)) return fail(FP8G_ERR_ALIGN, "A, B and D must be 16-byte aligned");
    if (!aligned4(scale_a) || !aligned4(scale_b) || !aligned4(masked_m))
        return fail(FP8G_ERR_ALIGN, "scale arrays and masked_m must be 4-byte aligned");
    if (N % 8) return fail(FP8G_ERR_ALIGN, "N=%d: rows of D must stay 16-byte aligned (N %% 8 == 0)", N);
    const int64_t kb = cdiv(K, 128), nb = cdiv(N, 128);
    if (lds_a < cap || lds_b < kb) return fail(FP8G_ERR_STRIDE, "lds_a=%lld below cap=%d or lds_b=%lld below ceil(K/128)=%lld",
                                               (long long)lds_a, cap, (long long)lds_b, (long long)kb);
    if (lds_a % 4 || lds_b % 4) return fail(FP8G_ERR_ALIGN, "lds_a=%lld / lds_b=%lld not multiples of 4", (long long)lds_a, (long long)lds_b);
    if (kb * lds_a > INT32_MAX - 256 || nb * lds_b > INT32_MAX - 256)
        return fail(FP8G_ERR_STRIDE, "a group's scale array above 2^31 bytes");
    if ((st = check_device()) != FP8G_OK) return st;

    GemmParams p = {};
    p.A = static_cast<const uint8_t *>(A);
    p.B = static_cast<const uint8_t *>(B);
    p.D = static_cast<uint16_t *>(D);
    p.lda = K; p.ldb = K; p.ldd = N;
    p.a_gstride = (int64_t)cap * K;
    p.b_gstride = (int64_t)N * K;
    p.d_gstride = (int64_t)cap * N;
    p.M = cap; p.N = N; p.K = K; p.G = G; p.cap = cap;
    p.masked_m = masked_m;
    p.sfa = scale_a; p.sfb = scale_b; p.lds_sa = lds_a; p.lds_sb = lds_b;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (plan.variant == V_SWAP) {
        p.tiles_m = 1;
        p.tiles_n = (int)cdiv(N, plan.tile_n);
        return launch_swap<fp8g::MODE_MASKED, fp8g::SCALE_BLOCK>(plan, a_dtype, b_dtype, p, s);
    }
    p.tiles_m = (int)cdiv(cap, 128);
    p.tiles_n = (int)cdiv(N, 256);
    return launch_tile128<fp8g::MODE_MASKED, fp8g::SCALE_BLOCK>(a_dtype, b_dtype, p,
                                                                dim3((unsigned)(p.tiles_m * p.tiles_n), (unsigned)G), s);
}

int fp8_grouped_gemm_contig(const void *A, int a_dtype, const void *B, int b_dtype, const float *scale_a,
                            const float *scale_b, const int32_t *grp_idx, void *D, int M_total, int G, int N, int K,
                            void *stream) {
    if (!dtype_ok(a_dtype) || !dtype_ok(b_dtype)) return fail(FP8G_ERR_DTYPE, "dtypes %d, %d", a_dtype, b_dtype);
    if (G < 0 || M_total < 0) return fail(FP8G_ERR_SHAPE, "negative G=%d or M_total=%d", G, M_total);
    fp8g_plan plan;
    int st = plan_impl(2, M_total, N, K, G, 0, &plan);
    if (st != FP8G_OK) return st;
    if (plan.variant == V_NONE) return ok();
    if ((K > 0 && (!A || !B)) || !D || !scale_a || !scale_b || !grp_idx)
        return fail(FP8G_ERR_NULL, "A, B (unless K = 0), D, scale_a, scale_b and grp_idx are required");
    if (!aligned16(A) || !aligned16(B) || !aligned16(D)) return fail(FP8G_ERR_ALIGN, "A, B and D must be 16-byte aligned");
    if (!aligned4(scale_a) || !aligned4(scale_b) || !aligned4(grp_idx)) return fail(FP8G_ERR_ALIGN, "scales and grp_idx must be 4-byte aligned");
    if (N % 8) return fail(FP8G_ERR_ALIGN, "N=%d: rows of D must stay 16-byte aligned (N %% 8 == 0)", N);
    if ((st = check_device()) != FP8G_OK) return st;

    GemmParams p = {};
    p.A = static_cast<const uint8_t *>(A);
    p.B = static_cast<const uint8_t *>(B);
    p.D = static_cast<uint16_t *>(D);
    p.lda = K; p.ldb = K; p.ldd = N;
    p.b_gstride = (int64_t)N * K;
    p.M = M_total; p.N = N; p.K = K; p.G = G; p.cap = M_total;
    p.scale_a = scale_a; p.scale_b = scale_b; p.grp_idx = grp_idx;
    hipStream_t s = static_cast<hipStream_t>(stream);
    p.tiles_m = (int)cdiv(M_total, 2 * kContigAlign);
    p.tiles_n = (int)cdiv(N, 256);
    // 8 waves: measured faster than the 4-wave kernel here (every expert's
    // weights stream from HBM); block scales are the other way round.
    return launch_ring<256, 256, T256_WM, T256_WN, T256_ST, T256_BK, fp8g::MODE_CONTIG, fp8g::SCALE_TENSOR>(
        a_dtype, b_dtype, p, dim3((unsigned)plan.workgroups), s);
}

int fp8_gemm_nt_blockscaled(const void *A, int64_t lda, int a_dtype, const void *B, int64_t ldb, int b_dtype,
                            const uint8_t *scale_a, int64_t lds_a, const uint8_t *scale_b, int64_t lds_b,
                            void *D, int64_t ldd, int M, int N, int K, void *stream) {
    if (!dtype_ok(a_dtype) || !dtype_ok(b_dtype)) return fail(FP8G_ERR_DTYPE, "dtypes %d, %d", a_dtype, b_dtype);
    fp8g_plan plan;
    int st = plan_impl(3, M, N, K, 1, 0, &plan);
    if (st != FP8G_OK) return st;
    if (plan.variant == V_NONE) return ok();
    if ((K > 0 && (!A || !B || !scale_a || !scale_b)) || !D)
        return fail(FP8G_ERR_NULL, "A, B, scale_a, scale_b (unless K = 0) and D are required");
    if (!aligned16(A) || !aligned16(B) || !aligned16(D)) return fail(FP8G_ERR_ALIGN, "A, B and D must be 16-byte aligned");
    if (!aligned4(scale_a) || !aligned4(scale_b)) return fail(FP8G_ERR_ALIGN, "scale arrays must be 4-byte aligned");
    if (lda < K || ldb < K) return fail(FP8G_ERR_STRIDE, "lda=%lld / ldb=%lld below K=%d", (long long)lda, (long long)ldb, K);
    if (lda % 16 || ldb % 16) return fail(FP8G_ERR_ALIGN, "lda=%lld / ldb=%lld not multiples of 16 bytes", (long long)lda, (long long)ldb);
    if (lda > kMaxRowStride || ldb > kMaxRowStride) return fail(FP8G_ERR_STRIDE, "row stride above %lld bytes", (long long)kMaxRowStride);
    if (ldd < N) return fail(FP8G_ERR_STRIDE, "ldd=%lld below N=%d", (long long)ldd, N);
    if (ldd % 8) return fail(FP8G_ERR_ALIGN, "ldd=%lld not a multiple of 8 elements", (long long)ldd);
    const int64_t kb = cdiv(K, 128), nb = cdiv(N, 128);
    if (lds_a < M || lds_b < kb) return fail(FP8G_ERR_STRIDE, "lds_a=%lld below M=%d or lds_b=%lld below ceil(K/128)=%lld",
                                             (long long)lds_a, M, (long long)lds_b, (long long)kb);
    if (lds_a % 4 || lds_b % 4) return fail(FP8G_ERR_ALIGN, "lds_a=%lld / lds_b=%lld not multiples of 4", (long long)lds_a, (long long)lds_b);
    if (kb * lds_a > INT32_MAX - 256 || nb * lds_b > INT32_MAX - 256)
        return fail(FP8G_ERR_STRIDE, "scale arrays above 2^31 bytes");
    if ((st = check_device()) != FP8G_OK) return st;

    GemmParams p = {};
    p.A = static_cast<const uint8_t *>(A);
    p.B = static_cast<const uint8_t *>(B);
    p.D = static_cast<uint16_t *>(D);
    p.lda = lda; p.ldb = ldb; p.ldd = ldd;
    p.M = M; p.N = N; p.K = K; p.G = 1; p.cap = M;
    p.sfa = scale_a; p.sfb = scale_b; p.lds_sa = lds_a; p.lds_sb = lds_b;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int fa = a_dtype, fb = b_dtype;
    const dim3 grid((unsigned)plan.workgroups);
    if (plan.variant == V_DECODE) {
        SplitWs ws;
        if ((st = decode_workspace(plan, s, ws)) != FP8G_OK) return st;
        return launch_decode<fp8g::SCALE_BLOCK>(plan, fa, fb, p, ws, s);
    }
    p.tiles_m = (int)cdiv(M, plan.tile_m);
    p.tiles_n = (int)cdiv(N, plan.tile_n);
    if (plan.variant == V_TILE_256x256) return launch_tile256<fp8g::MODE_DENSE, fp8g::SCALE_BLOCK>(fa, fb, p, grid, s);
    return launch_tile128<fp8g::MODE_DENSE, fp8g::SCALE_BLOCK>(fa, fb, p, grid, s);
}

int fp8_gemm_nt_channelwise(const void *A, int64_t lda, int a_dtype, const void *B, int64_t ldb, int b_dtype,
                            const float *scale_a, const float *scale_b, const float *bias,
                            void *D, int64_t ldd, int M, int N, int K, void *stream) {
    if (!dtype_ok(a_dtype) || !dtype_ok(b_dtype)) return fail(FP8G_ERR_DTYPE, "dtypes %d, %d", a_dtype, b_dtype);
    fp8g_plan plan;
    int st = plan_impl(0, M, N, K, 1, 0, &plan);
    if (st != FP8G_OK) return st;
    if (plan.variant == V_NONE) return ok();
    if ((K > 0 && (!A || !B)) || !D) return fail(FP8G_ERR_NULL, "A, B (unless K = 0) and D are required");
    if (!aligned16(A) || !aligned16(B) || !aligned16(D)) return fail(FP8G_ERR_ALIGN, "A, B and D must be 16-byte aligned");
    if (!aligned4(scale_a) || !aligned16(scale_b) || !aligned16(bias))
        return fail(FP8G_ERR_ALIGN, "scale_a must be 4-byte, scale_b and bias 16-byte aligned");
    if (lda < K || ldb < K) return fail(FP8G_ERR_STRIDE, "lda=%lld / ldb=%lld below K=%d", (long long)lda, (long long)ldb, K);
    if (lda % 16 || ldb % 16) return fail(FP8G_ERR_ALIGN, "lda=%lld / ldb=%lld not multiples of 16 bytes", (long long)lda, (long long)ldb);
    if (lda > kMaxRowStride || ldb > kMaxRowStride) return fail(FP8G_ERR_STRIDE, "row stride above %lld bytes", (long long)kMaxRowStride);
    if (ldd < N) return fail(FP8G_ERR_STRIDE, "ldd=%lld below N=%d", (long long)ldd, N);
    if (ldd % 8) return fail(FP8G_ERR_ALIGN, "ldd=%lld not a multiple of 8 elements", (long long)ldd);
    if ((st = check_device()) != FP8G_OK) return st;

    GemmParams p = {};
    p.A = static_cast<const uint8_t *>(A);
    p.B = static_cast<const uint8_t *>(B);
    p.D = static_cast<uint16_t *>(D);
    p.lda = lda; p.ldb = ldb; p.ldd = ldd;
    p.M = M; p.N = N; p.K = K; p.G = 1; p.cap = M;
    p.ch_sa = scale_a; p.ch_sb = scale_b; p.bias = bias;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int fa = a_dtype, fb = b_dtype;
    const dim3 grid((unsigned)plan.workgroups);
    if (plan.variant == V_DECODE) {
        SplitWs ws;
        if ((st = decode_workspace(plan, s, ws)) != FP8G_OK) return st;
        return launch_decode<fp8g::SCALE_CHANNEL>(plan, fa, fb, p, ws, s);
    }
    p.tiles_m = (int)cdiv(M, plan.tile_m);
    p.tiles_n = (int)cdiv(N, plan.tile_n);
    if (plan.variant == V_TILE_256x256) return launch_tile256<fp8g::MODE_DENSE, fp8g::SCALE_CHANNEL>(fa, fb, p, grid, s);
    if (plan.variant == V_TILE_256x192 || plan.variant == V_TILE_256x224)
        return launch_tile256_narrow<fp8g::SCALE_CHANNEL>(plan.variant, fa, fb, p, grid, s);
    return launch_tile128<fp8g::MODE_DENSE, fp8g::SCALE_CHANNEL>(fa, fb, p, grid, s);
}

int fp8_grouped_gemm_contig_blockscaled(const void *A, int a_dtype, const void *B, int b_dtype,
                                        const uint8_t *scale_a, int64_t lds_a, const uint8_t *scale_b, int64_t lds_b,
                                        const int32_t *grp_idx, void *D, int M_total, int G, int N, int K,
                                        void *stream) {
    if (!dtype_ok(a_dtype) || !dtype_ok(b_dtype)) return fail(FP8G_ERR_DTYPE, "dtypes %d, %d", a_dtype, b_dtype);
    if (G < 0 || M_total < 0) return fail(FP8G_ERR_SHAPE, "negative G=%d or M_total=%d", G, M_total);
    fp8g_plan plan;
    int st = plan_impl(5, M_total, N, K, G, 0, &plan);
    if (st != FP8G_OK) return st;
    if (plan.variant == V_NONE) return ok();
    if ((K > 0 && (!A || !B || !scale_a || !scale_b)) || !D || !grp_idx)
        return fail(FP8G_ERR_NULL, "A, B, scale_a, scale_b (unless K = 0), D and grp_idx are required");
    if (!aligned16(A) || !aligned16(B) || !aligned16(D)) return fail(FP8G_ERR_ALIGN, "A, B and D must be 16-byte aligned");
    if (!aligned4(scale_a) || !aligned4(scale_b) || !aligned4(grp_idx))
        return fail(FP8G_ERR_ALIGN, "scale arrays and grp_idx must be 4-byte aligned");
    if (N % 8) return fail(FP8G_ERR_ALIGN, "N=%d: rows of D must stay 16-byte aligned (N %% 8 == 0)", N);
    const int64_t kb = cdiv(K, 128), nb = cdiv(N, 128);
    if (lds_a < M_total || lds_b < kb)
        return fail(FP8G_ERR_STRIDE, "lds_a=%lld below M_total=%d or lds_b=%lld below ceil(K/128)=%lld",
                    (long long)lds_a, M_total, (long long)lds_b, (long long)kb);
    if (lds_a % 4 || lds_b % 4) return fail(FP8G_ERR_ALIGN, "lds_a=%lld / lds_b=%lld not multiples of 4", (long long)lds_a, (long long)lds_b);
    if (kb * lds_a > INT32_MAX - 256 || nb * lds_b > INT32_MAX - 256)
        return fail(FP8G_ERR_STRIDE, "scale array above 2^31 bytes");
    if ((st = check_device()) != FP8G_OK) return st;

    GemmParams p = {};
    p.A = static_cast<const uint8_t *>(A);
    p.B = static_cast<const uint8_t *>(B);
    p.D = static_cast<uint16_t *>(D);
    p.lda = K; p.ldb = K; p.ldd = N;
    p.b_gstride = (int64_t)N * K;
    p.M = M_total; p.N = N; p.K = K; p.G = G; p.cap = M_total;
    p.grp_idx = grp_idx;
    p.sfa = scale_a; p.sfb = scale_b; p.lds_sa = lds_a; p.lds_sb = lds_b;
    hipStream_t s = static_cast<hipStream_t>(stream);
    p.tiles_m = (int)cdiv(cdiv(M_total, kContigAlign), 2);
    p.tiles_n = (int)cdiv(N, 256);
    return launch_tile16<256, 2, fp8g::MODE_CONTIG, fp8g::SCALE_BLOCK>(a_dtype, b_dtype, p,
                                                                     dim3((unsigned)plan.workgroups), s);
}

}  // extern "C"
