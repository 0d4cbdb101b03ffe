// C ABI of the gfx950 FP8 GEMM library: argument validation, shape-class
// dispatch (including the swap-AB choice) and kernel launch on the caller's
// stream.  See include/fp8_gemm.h for the contract of every entry point.
#include <hip/hip_runtime.h>

#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

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
constexpr int kSwapMaxM = 64;                                  // swap-AB threshold on the token count
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

// Decode kernel: 16 weight rows per workgroup, or 32 where that still gives
// at least 256 workgroups.  Every workgroup reads all M x K token bytes, so
// fewer, larger row blocks cut the token traffic per CU (N = 14336: 896
// workgroups of 16 rows read 3.5 copies of the tokens per CU, 448 of 32 rows
// 1.75).
int decode_rows_for(int64_t n) { return cdiv(n, 2 * kDecodeRows) >= 256 ? 2 * kDecodeRows : kDecodeRows; }

// Swapped streaming kernel: 128 weight rows per wave (512 per workgroup), or
// 64 when that would leave CUs idle (16 groups of N = 4096: 128 workgroups
// of 512 rows ran at 4.4 TB/s).
int swap_wave_rows(int64_t groups, int64_t n) { return groups * cdiv(n, 4 * kSwapWaveRows) >= 256 ? kSwapWaveRows : kSwapWaveRows / 2; }

int token_blocks_for(int m) {
    if (m <= 16) return 1;
    if (m <= 32) return 2;
    return 4;
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

int tile_m_of(int variant) { return variant == V_TILE_128x256 ? 128 : 256; }
int tile_n_of(int variant) { return variant == V_TILE_256x192 ? 192 : variant == V_TILE_256x224 ? 224 : 256; }

int plan_impl(int op, int m, int n, int k, int groups, int expected_m, fp8g_plan *out) {
    memset(out, 0, sizeof *out);
    if (m < 0 || n < 0 || k < 0 || groups < 0) return fail(FP8G_ERR_SHAPE, "negative size (m=%d n=%d k=%d groups=%d)", m, n, k, groups);
    // K in bytes: 16-byte chunks of the ring (BF16: 2 bytes per element)
    const int64_t kbytes = op == 4 ? 2 * (int64_t)k : k;
    if (kbytes % 16 != 0) return fail(FP8G_ERR_SHAPE, "K=%d is not a multiple of %d", k, op == 4 ? 8 : 16);
    if (kbytes > kMaxRowStride) return fail(FP8G_ERR_SHAPE, "K=%d exceeds the row-stride limit %lld bytes", k, (long long)kMaxRowStride);
    if (op == 0) {
        if (m == 0 || n == 0) return ok();
        if (m <= kSwapMaxM) {
            out->variant = V_DECODE;
            out->tile_m = 16 * token_blocks_for(m);
            out->tile_n = decode_rows_for(n);
            out->token_blocks = token_blocks_for(m);
            out->workgroups = cdiv(n, out->tile_n);
        } else {
            out->variant = pick_dense_tile(m, n, true);
            out->tile_m = tile_m_of(out->variant);
            out->tile_n = tile_n_of(out->variant);
            out->workgroups = cdiv(m, out->tile_m) * cdiv(n, out->tile_n);
        }
        return ok();
    }
    if (op == 1) {
        if (expected_m < 0 || expected_m > m)
            return fail(FP8G_ERR_ARG, "expected_m=%d outside [0, cap=%d]", expected_m, m);
        if (groups == 0 || m == 0 || n == 0) return ok();
        const int hint = expected_m > 0 ? expected_m : m;
        if (hint <= kSwapMaxM) {
            out->variant = V_SWAP;
            out->tile_m = 16 * token_blocks_for(hint);
            out->tile_n = 4 * swap_wave_rows(groups, n);
            out->token_blocks = token_blocks_for(hint);
            out->workgroups = (int64_t)groups * cdiv(n, out->tile_n);
        } else {
            out->variant = V_TILE_128x256;
            out->tile_m = 128;
            out->tile_n = 256;
            out->workgroups = (int64_t)groups * cdiv(m, 128) * cdiv(n, 256);
        }
        return ok();
    }
    if (op == 2) {
        if (m == 0 || n == 0) return ok();
        if (groups == 0) return fail(FP8G_ERR_SHAPE, "G=0 with M_total=%d rows", m);
        // 256-row tiles, then one workgroup per tile for its second 128-row
        // block, which computes only when that block's expert differs.
        out->variant = V_TILE_256x256;
        out->tile_m = 2 * kContigAlign;
        out->tile_n = 256;
        out->workgroups = 2 * cdiv(m, 2 * kContigAlign) * cdiv(n, 256);
        return ok();
    }
    if (op == 3) {
        // Block-scaled dense: the decode kernel for few tokens, else the tiled
        // kernel (block scales applied per 128-byte K step of its ring).
        if (m == 0 || n == 0) return ok();
        if (m <= kSwapMaxM) {
            out->variant = V_DECODE;
            out->tile_m = 16 * token_blocks_for(m);
            out->tile_n = decode_rows_for(n);
            out->token_blocks = token_blocks_for(m);
            out->workgroups = cdiv(n, out->tile_n);
            return ok();
        }
        out->variant = pick_dense_tile(m, n, false);
        out->tile_m = tile_m_of(out->variant);
        out->tile_n = 256;
        out->workgroups = cdiv(m, out->tile_m) * cdiv(n, 256);
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
// 224 and 256 x 192 for dense FP8 without block scales).  Dense FP8 (any scale
// form) runs on 4 waves and the 16x16x128 instruction (2-slot ring, 128 KB of
// LDS, for 256 rows; 3-slot, 144 KB, for 128 rows); BF16 and the grouped forms
// on 8 waves and 32x32x64 (4 x 2 waves and a 2-slot ring for 256 rows, 2 x 4
// and 3 slots for 128).
template <int MODE, int SCL = 0>
int launch_tile256(int fa, int fb, const GemmParams &p, dim3 grid, hipStream_t s) {
    if constexpr (MODE == fp8g::MODE_DENSE) {
        if (fa != fp8g::FMT_BF16) return launch_tile16<256, 2, MODE, SCL>(fa, fb, p, grid, s);
        if constexpr (SCL == fp8g::SCALE_TENSOR)
            return launch_ring<256, 256, T256_WM, T256_WN, T256_ST, T256_BK, MODE, SCL, true>(fa, fb, p, grid, s);
        else
            return fail(FP8G_ERR_ARG, "BF16 operands take no scales");
    } else {
        return launch_ring<256, 256, T256_WM, T256_WN, T256_ST, T256_BK, MODE, SCL>(fa, fb, p, grid, s);
    }
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
    if (plan.tile_n == 4 * kSwapWaveRows) return launch_swap_wr<kSwapWaveRows, MODE, SCL>(plan.token_blocks, fa, fb, p, grid, s);
    return launch_swap_wr<kSwapWaveRows / 2, MODE, SCL>(plan.token_blocks, fa, fb, p, grid, s);
}

// Decode kernel: 4 waves per workgroup and per-wave LDS rings, as deep as fits
// in 80 KB so that two workgroups share a CU: 5, 3 or 2 steps for 1, 2 or 4
// token blocks with one weight block, 3, 2, 2 with two (the last needs 96 KB:
// one workgroup per CU).  Measured best against 8 waves and deeper rings with
// one workgroup per CU.  Block scales add 512 bytes per slot.
constexpr int kDecodeWaves = 4;

template <int RB, int CB, int SCL>
int launch_decode_cb(int fa, int fb, const GemmParams &p, dim3 grid, hipStream_t s) {
    constexpr int D = RB == 1 ? (CB == 1 ? 5 : (CB == 2 ? 3 : 2)) : (CB == 1 ? 3 : 2);
    const dim3 block(64 * kDecodeWaves);
#define FP8G_DEC(FA, FB) \
    hipLaunchKernelGGL((fp8g::decode_kernel<kDecodeWaves, RB, CB, FA, FB, D, SCL>), grid, block, 0, s, p)
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

template <int SCL>
int launch_decode(const fp8g_plan &plan, int fa, int fb, const GemmParams &p, hipStream_t s) {
    const dim3 grid((unsigned)plan.workgroups);
    if (plan.tile_n == 2 * kDecodeRows) return launch_decode_rb<2, SCL>(plan.token_blocks, fa, fb, p, grid, s);
    return launch_decode_rb<1, SCL>(plan.token_blocks, fa, fb, p, grid, s);
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

int fp8_gemm_nt(const void *A, int64_t lda, int a_dtype, const void *B, int64_t ldb, int b_dtype,
                const float *scale_a, const float *scale_b, void *D, int64_t ldd, int M, int N, int K,
                void *stream) {
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
    if (plan.variant == V_DECODE)
        return launch_decode<fp8g::SCALE_TENSOR>(plan, fa, fb, p, s);
    p.tiles_m = (int)cdiv(M, plan.tile_m);
    p.tiles_n = (int)cdiv(N, plan.tile_n);
    const dim3 grid((unsigned)plan.workgroups);
    if (plan.variant == V_TILE_256x256) return launch_tile256<fp8g::MODE_DENSE>(fa, fb, p, grid, s);
    if (plan.variant == V_TILE_256x192 || plan.variant == V_TILE_256x224)
        return launch_tile256_narrow<fp8g::SCALE_TENSOR>(plan.variant, fa, fb, p, grid, s);
    return launch_tile128<fp8g::MODE_DENSE>(fa, fb, p, grid, s);
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
    return launch_tile256<fp8g::MODE_CONTIG>(a_dtype, b_dtype, p, dim3((unsigned)plan.workgroups), s);
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
    if (plan.variant == V_DECODE) return launch_decode<fp8g::SCALE_BLOCK>(plan, fa, fb, p, s);
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
    if (plan.variant == V_DECODE) return launch_decode<fp8g::SCALE_CHANNEL>(plan, fa, fb, p, s);
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
    int st = plan_impl(2, M_total, N, K, G, 0, &plan);
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
    p.tiles_m = (int)cdiv(M_total, 2 * kContigAlign);
    p.tiles_n = (int)cdiv(N, 256);
    return launch_tile256<fp8g::MODE_CONTIG, fp8g::SCALE_BLOCK>(a_dtype, b_dtype, p, dim3((unsigned)plan.workgroups), s);
}

}  // extern "C"
