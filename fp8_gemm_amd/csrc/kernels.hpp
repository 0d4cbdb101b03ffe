// gfx950 FP8 GEMM kernels.
//
// The kernels compute D = bf16(sa * sb * A . B^T) with A [m x K] (tokens) and
// B [n x K] (weights), both K-contiguous ("nt"), and put B's rows on the
// matrix-core instruction's first (row) operand and A's rows on its second
// (column) operand.  Each lane's accumulator registers then hold four
// consecutive output columns n of one output row m, so the epilogue writes
// 8-byte packed BF16 runs straight from registers.
//
//   tile16_kernel  LDS-tiled, 256 x 256, 128 x 256, 256 x 224 or 256 x 192
//                  output tile per workgroup of 4 waves on v_mfma 16x16x128, K in steps of 128
//                  bytes, both operand tiles staged through a direct-to-LDS,
//                  XOR-swizzled ring.  Dense FP8 (M > 64) with per-tensor,
//                  per-channel or block scales; contiguous grouped FP8 (also
//                  block-scaled) on run-aligned 256 x 256 tiles.
//   ring_kernel    the same ring with 8 waves on v_mfma 32x32x64, BM x BN
//                  = 256 x 256 or 128 x 256: masked grouped with more than 192
//                  rows per group (also block-scaled), and the BF16 comparison
//                  path (same bytes, two v_mfma 32x32x16 BF16 per fragment).
//   swap_kernel    streaming "swap-AB" form for few tokens: each wave streams
//                  its own weight rows (every weight byte is used by exactly
//                  one wave) through a private LDS ring into the 16x16x128
//                  operand layout; tokens ride on the 16-wide column side in
//                  blocks of 16.  Masked grouped decode.
//   decode_kernel  the same idea for the dense form with M <= 64: 4 waves
//                  split K over 16 weight rows per workgroup; weights and
//                  tokens are copied line by line into per-wave LDS rings and
//                  read back in the 16x16x128 layout; the waves' partial sums
//                  are added through LDS.
//
// "DeepGEMM: FP8 matrix-multiply kernels on Hopper Tensor Cores" is the prior
// art for the tiled form (section 2.3 three-level tiling, section 3.3 double
// buffering, section 4.2 swizzled on-chip layout, section 6.3 clipping the last
// K block); "One transpose, half the compute: the DeepSeek SwapAB story"
// (sections 1.1, 3.2-3.3) for putting the weights on the instruction's rigid
// side and shrinking the token side to the valid rows.
#pragma once

#include "device_common.hpp"

namespace fp8g {

enum { MODE_DENSE = 0, MODE_MASKED = 1, MODE_CONTIG = 2 };
// Scale modes of the dense form: one scale per tensor, E8M0 block scales per
// 128-element K block, or a scale per row of A and a scale and bias per output
// channel applied in the epilogue.
enum { SCALE_TENSOR = 0, SCALE_BLOCK = 1, SCALE_CHANNEL = 2 };

struct GemmParams {
    const uint8_t *A;          // tokens: [m x K] rows of lda bytes (per group: + g * a_gstride)
    const uint8_t *B;          // weights: [n x K] rows of ldb bytes (per group: + g * b_gstride)
    uint16_t *D;               // BF16 [m x N], ldd elements (per group: + g * d_gstride)
    int64_t lda, ldb, ldd;
    int64_t a_gstride, b_gstride, d_gstride;
    int M, N, K, G, cap;
    const float *scale_a;      // 1 float
    const float *scale_b;      // 1 float (dense) or G floats (grouped)
    const int32_t *masked_m;   // masked: [G]
    const int32_t *grp_idx;    // contiguous: [M]
    int tiles_m, tiles_n;      // tile grid of one group
    // Block scales (block-scaled dense form): E8M0 codes; sfa[kb * lds_sa + m]
    // scales row m over K block kb (128 elements), sfb[nb * lds_sb + kb] rows
    // 128 nb .. 128 nb + 127 of B over K block kb.
    const uint8_t *sfa, *sfb;
    int64_t lds_sa, lds_sb;
    // Per-channel form: row scales of A [M], channel scales [N] and bias [N]
    // (each may be NULL: 1, 1, 0).
    const float *ch_sa, *ch_sb, *bias;
    // Few-token form with K split over workgroups (splits > 1): `splits`
    // workgroups per block of weight rows take `ksteps` 128-byte K steps each,
    // leave their FP32 partial sums in ws, and count their arrivals in
    // cnt[kCountStride * block]; the last to arrive adds the partial sums in
    // split order.
    float *ws;
    int *cnt;
    int splits, ksteps;
};

// Ints per arrival count of the split-K workspace: one 128-byte line each.
constexpr int kCountStride = 32;

// Epilogue terms of the per-channel form for four consecutive output channels
// n .. n+3: their scales and biases.  Channels at or past N take scale 0 and
// bias 0 (they are not stored).
__device__ __forceinline__ void channel_terms(const GemmParams &p, int n, float (&s4)[4], float (&b4)[4]) {
    if (n + 4 <= p.N) {
        if (p.ch_sb) {
            const v4f v = *reinterpret_cast<const v4f *>(p.ch_sb + n);
            s4[0] = v[0]; s4[1] = v[1]; s4[2] = v[2]; s4[3] = v[3];
        } else {
            s4[0] = s4[1] = s4[2] = s4[3] = 1.0f;
        }
        if (p.bias) {
            const v4f v = *reinterpret_cast<const v4f *>(p.bias + n);
            b4[0] = v[0]; b4[1] = v[1]; b4[2] = v[2]; b4[3] = v[3];
        } else {
            b4[0] = b4[1] = b4[2] = b4[3] = 0.0f;
        }
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const bool in = n + e < p.N;
            s4[e] = in ? (p.ch_sb ? p.ch_sb[n + e] : 1.0f) : 0.0f;
            b4[e] = in && p.bias ? p.bias[n + e] : 0.0f;
        }
    }
}

// ---------------------------------------------------------------------------
// Tile index -> (tm, tn) for the tiled kernel (dense and contiguous forms).
//
// Workgroups are dispatched in index order, round-robin over the 8 XCDs
// (workgroup w runs on XCD w % 8), and each XCD has its own L2.  Logical tiles
// are ordered in bands of kGroupM tile-rows (column by column inside a band),
// so consecutive logical tiles share few operand panels, and the remap gives
// each XCD runs of consecutive logical tiles:
//   CHUNKED = false: XCD x owns the x-th eighth of all tiles (for 4096^3 with
//     256 x 256 tiles, a 4 x 8 block of tiles: 12 panels instead of 64);
//   CHUNKED = true: chunks of kXcdChunk tiles (one XCD's worth of CUs) go to
//     the XCDs in turn, so the whole chip works on one window of consecutive
//     chunks at a time.  That keeps the working set small enough for the
//     last-level (Infinity) cache when the operands are far larger than it, as
//     in the contiguous grouped form where every expert brings its own
//     weights (measured 14% faster there, 2-3% slower for large dense shapes
//     whose weights stay cached either way).
// ---------------------------------------------------------------------------
constexpr int kXcds = 8;
constexpr int kXcdChunk = 32;
constexpr int kGroupM = 4;

template <bool CHUNKED>
__device__ __forceinline__ void tile_coords(int wg, int tiles_m, int tiles_n, int &tm, int &tn) {
    const int nt = tiles_m * tiles_n;
    int t = wg;
    if (CHUNKED) {
        constexpr int round = kXcds * kXcdChunk;
        if (wg < (nt / round) * round) {
            // wg = 8 k + x: the k-th workgroup of XCD x
            const int x = wg % kXcds, k = wg / kXcds;
            t = ((k / kXcdChunk) * kXcds + x) * kXcdChunk + k % kXcdChunk;
        }
    } else {
        const int per_xcd = nt / kXcds;
        if (wg < per_xcd * kXcds) t = (wg % kXcds) * per_xcd + wg / kXcds;
    }
    const int band = kGroupM * tiles_n;
    const int b = t / band;
    const int first_m = b * kGroupM;
    const int rows = min(kGroupM, tiles_m - first_m);
    const int r = t - b * band;
    tm = first_m + r % rows;
    tn = r / rows;
}

// ---------------------------------------------------------------------------
// Placement of one output tile of the tiled kernels (dense and masked forms):
// tile coordinates, group, first row and the valid rows and columns.  Returns
// false when the workgroup has nothing to compute (masked tile past the
// group's count).
// ---------------------------------------------------------------------------
struct TileSpot {
    int tm, tn, g, m0, rows_m, n0, rows_n, expert;
};

template <int BM, int BN, int MODE>
__device__ __forceinline__ bool place_tile(const GemmParams &p, int lane, TileSpot &t) {
    static_assert(MODE != MODE_CONTIG, "contiguous grouped form: place_contig_tile");
    (void)lane;
    t.g = 0;
    t.expert = 0;
    if (MODE == MODE_DENSE) {
        tile_coords<false>(blockIdx.x, p.tiles_m, p.tiles_n, t.tm, t.tn);
        t.m0 = t.tm * BM;
        t.rows_m = min(p.M - t.m0, BM);
    } else {
        t.tm = blockIdx.x / p.tiles_n;
        t.tn = blockIdx.x % p.tiles_n;
        t.g = blockIdx.y;
        t.m0 = t.tm * BM;
        const int mg = min(max(p.masked_m[t.g], 0), p.cap);
        if (t.m0 >= mg) return false;              // nothing valid in this tile: no load at all
        t.rows_m = min(mg - t.m0, BM);
        t.expert = t.g;
    }
    t.n0 = t.tn * BN;
    t.rows_n = min(p.N - t.n0, BN);
    return true;
}

// ---------------------------------------------------------------------------
// Paired tiles of the contiguous grouped form (8-wave kernel).
// A 256-row tile covers two 128-row blocks, each of at most one expert, and
// writes the rows of the expert of its first valid row.  A second set of
// workgroups, one per tile, appended to the grid, covers the second block
// when its expert differs: it computes that block alone (tile rows 128..255
// read zeros).  They come last in dispatch order, where the last partial
// wave of full tiles leaves CUs idle.  Measured against run-aligned tiles on
// the 8-wave kernel (fewer tiles, 4384 against 4480 tile passes on the
// 65536-row prefill, but up to two per workgroup): 1.72 against 1.78 ms.
// ---------------------------------------------------------------------------
__device__ __forceinline__ bool place_contig_pair(const GemmParams &p, int lane, TileSpot &t) {
    // the expert of a block of rows: that of its first row naming a valid
    // expert, -1 for a block of padding only
    auto first_expert = [&](int r0, int nrows) {
        for (int base = 0; base < nrows; base += 64) {
            const int r = base + lane;
            int e = -1;
            if (r < nrows) e = p.grp_idx[r0 + r];
            const bool ok = (e >= 0) && (e < p.G);
            const unsigned long long ball = __ballot(ok);
            if (ball) return __builtin_amdgcn_readfirstlane(__shfl(e, __builtin_ctzll(ball)));
        }
        return -1;
    };
    const int ntiles = p.tiles_m * p.tiles_n;
    t.g = 0;
    if ((int)blockIdx.x < ntiles) {
        tile_coords<true>(blockIdx.x, p.tiles_m, p.tiles_n, t.tm, t.tn);
        t.m0 = t.tm * 256;
        t.rows_m = min(p.M - t.m0, 256);
        t.expert = first_expert(t.m0, t.rows_m);
        if (t.expert < 0) return false;
    } else {
        const int w2 = blockIdx.x - ntiles;
        t.tm = w2 / p.tiles_n;
        t.tn = w2 % p.tiles_n;
        const int base = t.tm * 256;
        const int r2 = min(p.M - (base + 128), 128);
        if (r2 <= 0) return false;
        const int e1 = first_expert(base, min(p.M - base, 256));
        const int e2 = first_expert(base + 128, r2);
        if (e2 < 0 || e2 == e1) return false;
        t.m0 = base + 128;
        t.rows_m = r2;
        t.expert = e2;
    }
    t.n0 = t.tn * 256;
    t.rows_n = min(p.N - t.n0, 256);
    return true;
}

// ---------------------------------------------------------------------------
// Run-aligned tiles of the contiguous grouped form (4-wave kernel).
// The rows of one expert form a run of consecutive 128-row blocks.  Each run
// is covered by 256-row tiles from its first block on, the last one 128 rows
// when the run has an odd number of blocks, so no tile holds two experts and
// no block is computed twice.  A tile therefore starts at block b when b holds
// an expert and lies an even number of blocks past the start of its run.
// Workgroup slot t (of ceil(blocks / 2)) computes the tiles starting at blocks
// 2t and 2t + 1: zero, one or two of them.  Nothing is planned on the host, so
// the per-expert counts never leave the device.
// ---------------------------------------------------------------------------
// The expert of 128-row block b: that of its first row naming a valid expert,
// or -1 when the block is all padding.
__device__ __forceinline__ int contig_block_expert(const GemmParams &p, int b) {
    const int r0 = b * 128;
    const int n = min(128, p.M - r0);
    for (int i = 0; i < n; ++i) {
        const int e = p.grp_idx[r0 + i];
        if (e >= 0 && e < p.G) return e;
    }
    return -1;
}

// The tiles of this workgroup's slot t (blocks 2t, 2t + 1): found once, with
// one load per lane: lane l reads the expert of block 2t + 2 - l, which covers
// the next block after the slot (does a tile's run go on?) and 61 blocks
// before it (where does the run start?); longer runs take further rounds of 64
// blocks.  Returns, per pass (0: block 2t, 1: block 2t + 1), the tile's
// expert (or -1 when no tile starts there) and its number of blocks.
struct ContigSlot {
    int expert[2], nblk[2];
};

__device__ __forceinline__ ContigSlot contig_slot_tiles(const GemmParams &p, int lane, int t) {
    const int nb = (p.M + 127) / 128;
    const int b0 = 2 * t;
    auto expert_of = [&](int b) { return b >= 0 && b < nb ? contig_block_expert(p, b) : -1; };
    const int el = expert_of(b0 + 2 - lane);
    // blocks 2t + 2, 2t + 1, 2t
    const int e2 = __builtin_amdgcn_readfirstlane(__shfl(el, 0));
    const int e1 = __builtin_amdgcn_readfirstlane(__shfl(el, 1));
    const int e0 = __builtin_amdgcn_readfirstlane(__shfl(el, 2));
    // dist = blocks of expert e0 just before block 2t (its run start is 2t - dist)
    int dist = 0;
    if (e0 >= 0) {
        unsigned long long other = __ballot(lane >= 3 && el != e0);
        if (other) {
            dist = __builtin_ctzll(other) - 3;
        } else {
            dist = 61;
            for (int base = b0 - 62;; base -= 64) {
                const unsigned long long o = __ballot(expert_of(base - lane) != e0);
                if (o) {
                    dist += __builtin_ctzll(o);
                    break;
                }
                dist += 64;
            }
        }
    }
    ContigSlot s;
    // a tile starts at 2t when it holds an expert an even number of blocks
    // into its run; at 2t + 1 when it starts a run, or continues 2t's run
    // from an odd distance
    const bool at0 = e0 >= 0 && (dist & 1) == 0;
    const bool at1 = e1 >= 0 && (e1 != e0 || (dist & 1) == 1);
    // (uniform values, kept in scalar registers across the passes)
    s.expert[0] = __builtin_amdgcn_readfirstlane(at0 ? e0 : -1);
    s.nblk[0] = __builtin_amdgcn_readfirstlane(e1 == e0 ? 2 : 1);
    s.expert[1] = __builtin_amdgcn_readfirstlane(at1 ? e1 : -1);
    s.nblk[1] = __builtin_amdgcn_readfirstlane(e2 == e1 ? 2 : 1);
    return s;
}

// Placement of the tile of this workgroup's slot that starts at block
// 2t + pass, if any.
__device__ __forceinline__ bool place_contig_tile(const GemmParams &p, const ContigSlot &cs, int pass, TileSpot &t) {
    tile_coords<true>(blockIdx.x, p.tiles_m, p.tiles_n, t.tm, t.tn);
    const int e = cs.expert[pass];
    if (e < 0) return false;
    t.g = 0;
    t.expert = e;
    t.m0 = (2 * t.tm + pass) * 128;
    t.rows_m = min(p.M - t.m0, 128 * cs.nblk[pass]);
    t.n0 = t.tn * 256;
    t.rows_n = min(p.N - t.n0, 256);
    return true;
}

// Rows of a contiguous-form tile that belong to its expert: BM / 64 masks of
// 64 bits (bit r % 64 of mask r / 64 is row r of the tile), written to LDS
// with one ballot per 64 rows before the main loop (whose barriers publish
// them).  The epilogue's stores then test a bit; loading grp_idx for the row
// of every 16-byte chunk made each store wait on a global load.
template <int BM, int WAVES>
__device__ __forceinline__ void contig_row_mask(const GemmParams &p, const TileSpot &t, int wave, int lane,
                                                uint64_t *mask) {
    for (int g = wave; g < BM / 64; g += WAVES) {
        const int r = g * 64 + lane;
        const bool mine = r < t.rows_m && p.grp_idx[t.m0 + r] == t.expert;
        const uint64_t bits = __ballot(mine);
        if (lane == 0) mask[g] = bits;
    }
}

__device__ __forceinline__ bool row_in_mask(const uint64_t *mask, int r) { return (mask[r >> 6] >> (r & 63)) & 1; }

// Stored position of 16-byte chunk c of staged output row r (OCH chunks per
// row): c ^ (r % OCH) when OCH is a power of two, else (c + r) % OCH.  Either
// way a row keeps its chunks, and the rows one staging write touches land on
// different chunk positions.
template <int OCH>
__device__ __forceinline__ uint32_t stage_chunk(uint32_t c, uint32_t r) {
    return (OCH & (OCH - 1)) == 0 ? (c ^ (r % OCH)) : (c + r) % OCH;
}

// Store 8 BF16 outputs (16 bytes) of one row, of which the first nvalid are
// inside the output.  The dense form writes through the L2, so the next launch
// need not wait for the write-back of this output; the grouped forms' outputs
// are larger than the L2s and stream out regardless (measured 0.5% slower
// written through on the contiguous prefill).
template <int MODE>
__device__ __forceinline__ void store_chunk(uint16_t *dst, v4u v, int nvalid) {
    if (nvalid >= 8) {
        if (MODE == MODE_DENSE) store16_wt(dst, v);
        else *reinterpret_cast<v4u *>(dst) = v;
    } else if (nvalid > 0) {
        const uint16_t e[8] = {(uint16_t)(v[0] & 0xFFFFu), (uint16_t)(v[0] >> 16), (uint16_t)(v[1] & 0xFFFFu),
                               (uint16_t)(v[1] >> 16), (uint16_t)(v[2] & 0xFFFFu), (uint16_t)(v[2] >> 16),
                               (uint16_t)(v[3] & 0xFFFFu), (uint16_t)(v[3] >> 16)};
        for (int k = 0; k < nvalid; ++k) dst[k] = e[k];
    }
}

// Write a BF16 output tile staged in LDS (row r at r * BN * 2 bytes, 16-byte
// chunk c stored at stage_chunk(c, r)) with 16-byte stores of whole row
// segments; the contiguous form writes only the rows of the tile's expert
// (rowmask, see contig_row_mask).
template <int BM, int BN, int THREADS, int MODE>
__device__ __forceinline__ void store_staged(const GemmParams &p, const uint8_t *smem, int tid, const TileSpot &t,
                                             uint16_t *d_base, const uint64_t *rowmask = nullptr) {
    constexpr int OCH = BN / 8;
    constexpr int OUT_CHUNKS = BM * OCH;
    static_assert(OUT_CHUNKS % THREADS == 0, "staged tile splits evenly over the threads");
#pragma unroll 4
    for (int q = tid; q < OUT_CHUNKS; q += THREADS) {
        const int r = q / OCH;
        const int c = q % OCH;
        if (r >= t.rows_m) continue;
        const int m = t.m0 + r;
        if (MODE == MODE_CONTIG && !row_in_mask(rowmask, r)) continue;
        const int n = t.n0 + c * 8;
        const v4u v = *reinterpret_cast<const v4u *>(smem + r * (BN * 2) + stage_chunk<OCH>(c, r) * 16);
        store_chunk<MODE>(d_base + (int64_t)m * p.ldd + n, v, p.N - n);
    }
}

// ---------------------------------------------------------------------------
// LDS-tiled kernel with a direct-to-LDS ring.
// BM x BN tile (tokens x weights) per workgroup of WM x WN waves; each wave
// owns a TM x TN sub-tile of (TM/32) x (TN/32) 32x32 accumulator blocks.  K
// advances BK bytes per ring slot (BK/64 v_mfma 32x32x64 per accumulator
// block).  STAGES slots of (BM + BN) x BK bytes: the tile rows of step
// kt + STAGES - 1 are DMA'd from HBM straight into LDS while step kt is
// consumed, so STAGES - 1 steps of loads are in flight ("DeepGEMM on Hopper
// Tensor Cores", sections 3.3 and 4.3).  BK = 128 makes every DMA instruction
// read whole 128-byte row segments (8 rows x 128 B): with 64-byte segments
// each L2 line is fetched twice and streaming runs at two thirds of the rate.
// ---------------------------------------------------------------------------
template <int BK>
__device__ __forceinline__ uint32_t ring_key(uint32_t row) {
    // XOR key of the stored chunk index (see swz / swz64_key).
    return BK == 128 ? ((row & 7u) ^ ((row >> 3) & 1u)) : swz64_key(row);
}

template <int BM, int BN, int WM, int WN, int FA, int FB, int MODE, int STAGES, int BK, int SCL>
__global__ __launch_bounds__(64 * WM * WN, 1) void ring_kernel(GemmParams p) {
    constexpr bool BLK = SCL == SCALE_BLOCK;
    // BF16 operands: the ring moves bytes, so K, lda and ldb arrive in bytes
    // and only the instruction changes (see mfma32x32x16_bf16_part).
    constexpr bool BF = FA == FMT_BF16;
    static_assert(BF == (FB == FMT_BF16), "BF16 operands come in pairs");
    static_assert(!BF || (SCL == SCALE_TENSOR && MODE == MODE_DENSE), "BF16: dense form, no scales");
    constexpr int WAVES = WM * WN;
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int FM = TM / 32, FN = TN / 32;
    constexpr int KCH = BK / 16;                   // 16-byte chunks per tile row per slot
    constexpr int DROWS = 1024 / BK;               // tile rows covered by one 1 KB DMA instruction
    constexpr int SLOT = (BM + BN) * BK;           // bytes per ring slot
    constexpr int CHUNKS = SLOT / 1024;            // DMA instructions per slot
    constexpr int CPW = CHUNKS / WAVES;            // DMA instructions per wave per slot
    static_assert(BK == 64 || BK == 128, "K step");
    static_assert(CHUNKS % WAVES == 0 && CPW >= 1, "tile rows must split evenly over the waves");
    static_assert(FM >= 1 && FN >= 1 && TM % 32 == 0 && TN % 32 == 0, "wave tile");
    static_assert(STAGES >= 2 && CPW * (STAGES - 2) < 64, "ring depth");
    constexpr int STAGE_OUT = BM * BN * 2;         // BF16 output tile staged for the stores
    // Block scales (BLK): per ring slot, the step's scale of each tile row of A
    // (bytes 0..BM-1) and one dword per 128-row block of B (from byte 256).
    static_assert(!BLK || (BK == 128 && BM <= 256 && BN % 128 == 0), "block scales: 128-byte K steps");
    static_assert(SCL != SCALE_CHANNEL, "per-channel scales: tile16_kernel");
    constexpr int SCS = BLK ? 512 : 0;
    constexpr int RING = STAGES * (SLOT + SCS);
    constexpr int MASK_AT = RING > STAGE_OUT ? RING : STAGE_OUT;   // contiguous form: the tile's row mask
    constexpr int SMEM = MASK_AT + (MODE == MODE_CONTIG ? BM / 8 : 0);
    constexpr int THREADS = 64 * WAVES;
    constexpr int OCH = BN / 8;                    // 16-byte chunks per staged output row
    static_assert(OCH == 32 || OCH == 16, "staged row width");
    static_assert(MODE != MODE_CONTIG || (BM == 256 && BN == 256), "contiguous grouped form: 256 x 256 tiles");

    __shared__ __attribute__((aligned(1024))) uint8_t smem[SMEM];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave % WM;
    const int wn = wave / WM;

    // ---- tile coordinates and per-mode operand bases (64-bit arithmetic) ----
    TileSpot spot;
    if constexpr (MODE == MODE_CONTIG) {
        if (!place_contig_pair(p, lane, spot)) return;
    } else {
        if (!place_tile<BM, BN, MODE>(p, lane, spot)) return;
    }
    const int g = spot.g, m0 = spot.m0, rows_m = spot.rows_m, expert = spot.expert;
    const int n0 = spot.n0, rows_n = spot.rows_n;
    uint64_t *const rowmask = reinterpret_cast<uint64_t *>(smem + MASK_AT);
    if constexpr (MODE == MODE_CONTIG) contig_row_mask<BM, WAVES>(p, spot, wave, lane, rowmask);
    uint16_t *d_base = p.D + (MODE == MODE_MASKED ? (int64_t)g * p.d_gstride : 0);
    const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t *)smem;

    const uint8_t *a_base = p.A + (MODE == MODE_MASKED ? (int64_t)g * p.a_gstride : 0) + (int64_t)m0 * p.lda;
    const uint8_t *b_base = p.B + (int64_t)expert * p.b_gstride + (int64_t)n0 * p.ldb;
    const float sc = (SCL != SCALE_TENSOR || BF) ? 1.0f : p.scale_a[0] * p.scale_b[MODE == MODE_DENSE ? 0 : expert];

    // Rows past rows_m / rows_n fall outside the descriptors: the DMA writes
    // zeros for them and issues no memory transaction.
    const v4i srdA = make_srd(a_base, rows_bytes(rows_m, p.lda));
    const v4i srdB = make_srd(b_base, rows_bytes(rows_n, p.ldb));

    // ---- this wave's DMA chunks ----
    // Instruction q covers DROWS rows x BK bytes: A rows for q < BM / DROWS,
    // else B rows.  Lane l deposits LDS bytes [16 l, 16 l + 16) of it, i.e.
    // row l / KCH, stored chunk l % KCH; it loads logical chunk
    // (l % KCH) ^ key(row), so the LDS image is swizzled (see ring_key).  For
    // row = qq * DROWS + l / KCH (qq: the instruction's index within its
    // operand) the key depends on qq only through its parity, so a lane needs
    // two chunk choices and, per operand, two per-lane offsets; the rest of
    // the offset, qq * DROWS * ld, is the same for the whole wave.
    const uint32_t lrow_in = (uint32_t)lane / KCH;
    uint32_t dkc0 = (((uint32_t)lane % KCH) ^ ring_key<BK>(lrow_in)) & (KCH - 1);
    uint32_t dkc1 = (((uint32_t)lane % KCH) ^ ring_key<BK>(DROWS + lrow_in)) & (KCH - 1);
    dkc0 *= 16u;
    dkc1 *= 16u;
    uint32_t doA0 = lrow_in * (uint32_t)p.lda + dkc0, doA1 = lrow_in * (uint32_t)p.lda + dkc1;
    uint32_t doB0 = lrow_in * (uint32_t)p.ldb + dkc0, doB1 = lrow_in * (uint32_t)p.ldb + dkc1;
    const int nk = (p.K + BK - 1) / BK;
    auto issue_one = [&](int kt, int i) {
        const int q = wave * CPW + i;              // wave-uniform
        const bool isA = q < BM / DROWS;
        const int qq = isA ? q : q - BM / DROWS;
        const uint32_t k0 = (uint32_t)kt * BK;
        const uint32_t rowoff = (uint32_t)__builtin_amdgcn_readfirstlane(
            (int)((uint32_t)(qq * DROWS) * (uint32_t)(isA ? p.lda : p.ldb) + k0));
        const uint32_t kc = (qq & 1) ? dkc1 : dkc0;
        const uint32_t lo = (qq & 1) ? (isA ? doA1 : doB1) : (isA ? doA0 : doB0);
        const bool in = (kt < nk) && (int)(k0 + kc) < p.K;
        dma16(isA ? srdA : srdB, in ? lo + rowoff : kOobOffset,
              lds0 + (kt % STAGES) * SLOT + (uint32_t)q * 1024u);
    };
    // Block scales of step kt (wave 0): A's row scales, 4 rows per lane, and
    // the scale dword holding K block kt of each 128-row block of B.  Rows
    // past the scale array (or K blocks past the last) read zeros; rows past M
    // may read other in-range bytes, which only reach outputs not written.
    const int64_t sa_bytes = (int64_t)((p.K + 127) / 128) * p.lds_sa;
    const int64_t sb_bytes = (int64_t)((p.N + 127) / 128) * p.lds_sb;
    const v4i srdSA = BLK ? make_srd(p.sfa + (MODE == MODE_MASKED ? (int64_t)g * sa_bytes : 0), (uint32_t)sa_bytes)
                          : v4i{0, 0, 0, 0};
    // weight-block scales: per group (masked) or per expert (contiguous);
    // token-row scales: per group (masked) or by global row (contiguous)
    const int64_t sb_group = MODE == MODE_MASKED ? g : (MODE == MODE_CONTIG ? expert : 0);
    const v4i srdSB = BLK ? make_srd(p.sfb + sb_group * sb_bytes, (uint32_t)sb_bytes) : v4i{0, 0, 0, 0};
    const uint32_t scl_base = lds0 + STAGES * SLOT;
    auto issue_scales = [&](int kt) {
        if (!BLK || wave != 0) return;
        const uint32_t slot = scl_base + (uint32_t)(kt % STAGES) * SCS;
        const bool ka = (kt < nk) && 4 * lane < BM;
        dma4(srdSA, ka ? (uint32_t)(kt * p.lds_sa + m0 + 4 * lane) : kOobOffset, slot);
        const bool kb = (kt < nk) && lane < BN / 128;
        dma4(srdSB, kb ? (uint32_t)((n0 / 128 + lane) * p.lds_sb + (kt & ~3)) : kOobOffset, slot + 256);
    };
    constexpr int SCW = BLK ? 2 : 0;               // scale DMA instructions per step of wave 0
    // 256-row tiles (UNI): each wave copies one operand's rows, so, as in
    // tile16_kernel, a lane's offset within the tile is fixed per copy and
    // kept in a register, each step only moves the descriptor's base (and
    // shrinks its byte count) and M0 goes to the compiler as an operand.  The
    // lanes whose K chunk starts at or past K add kOobOffset (every lane,
    // past the last step, where the byte count is also 0).
    constexpr bool UNI = BK == 128 && (BM / DROWS) % CPW == 0;
    const bool wA = wave * CPW < BM / DROWS;       // wave-uniform
    uint32_t lo_q[CPW];
    if (UNI) {
#pragma unroll
        for (int i = 0; i < CPW; ++i) {
            const int qq = (wave * CPW + i) % (BM / DROWS);
            lo_q[i] = (uint32_t)(qq * DROWS + (int)lrow_in) * (uint32_t)(wA ? p.lda : p.ldb) + ((qq & 1) ? dkc1 : dkc0);
        }
    }
    const v4i srd0 = wA ? srdA : srdB;
    const uint64_t base0 = ((uint64_t)(uint32_t)srd0[1] << 32) | (uint32_t)srd0[0];
    v4i srdk = srd0;
    uint32_t lds_slot = 0, ko0 = 0, ko1 = 0;
    auto set_step = [&](int kd) {
        const uint64_t b = base0 + (uint64_t)kd * BK;
        srdk[0] = (int)(uint32_t)b;
        srdk[1] = (int)(uint32_t)(b >> 32);
        srdk[2] = kd < nk ? srd0[2] - kd * BK : 0;
        lds_slot = lds0 + (uint32_t)(kd % STAGES) * SLOT + (uint32_t)(wave * CPW) * 1024u;
        const int lim = p.K - kd * BK;
        ko0 = (int)dkc0 < lim ? 0u : kOobOffset;
        ko1 = (int)dkc1 < lim ? 0u : kOobOffset;
    };
    auto issue_fast = [&](int i) {   // CPW is even, so copy i's key parity is that of i
        dma16_m0(srdk, lo_q[i] + ((i & 1) ? ko1 : ko0), lds_slot + (uint32_t)i * 1024u);
    };
    auto issue = [&](int kt) {
        if (UNI) set_step(kt);
#pragma unroll
        for (int i = 0; i < CPW; ++i) {
            if (UNI) issue_fast(i);
            else issue_one(kt, i);
        }
        issue_scales(kt);
    };

    // ---- fragment read offsets ----
    // v_mfma 32x32x64 operands: lane l carries row l & 31 of its 32-row block
    // and K bytes [(l >> 5) * 32, +32) of each 64-byte K half h of the slot,
    // i.e. logical chunks 4 h + 2 (l >> 5) and 4 h + 2 (l >> 5) + 1.  Both
    // operands use the same K placement, so each dot product covers exactly
    // that K half.
    constexpr int KH = BK / 64;                    // MFMA K steps per slot
    const int lrow = lane & 31;
    const int khalf = lane >> 5;
    const uint32_t key = ring_key<BK>((uint32_t)lrow);   // blocks start at multiples of 32 rows
    uint32_t fo[KH][2];
#pragma unroll
    for (int h = 0; h < KH; ++h)
#pragma unroll
        for (int j = 0; j < 2; ++j)
            fo[h][j] = (uint32_t)lrow * BK + (((uint32_t)(4 * h + 2 * khalf + j) ^ key) & (KCH - 1)) * 16u;
    const uint32_t a_frag = (uint32_t)(wm * TM) * BK;
    const uint32_t b_frag = (uint32_t)BM * BK + (uint32_t)(wn * TN) * BK;

    v16f acc[FN][FM];
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j) acc[i][j] = (v16f){0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};

    // Fragments of one 64-deep K half: FN row-operand blocks (B rows) and FM
    // column-operand blocks (A rows), 32 bytes per lane each.
    auto read_frags = [&](v8i (&bf)[FN], v8i (&af)[FM], const uint8_t *slot, int h) {
#pragma unroll
        for (int f = 0; f < FN; ++f) {
            const uint8_t *r = slot + b_frag + f * 32 * BK;
            bf[f] = pack8(*reinterpret_cast<const v4u *>(r + fo[h][0]), *reinterpret_cast<const v4u *>(r + fo[h][1]));
        }
#pragma unroll
        for (int f = 0; f < FM; ++f) {
            const uint8_t *r = slot + a_frag + f * 32 * BK;
            af[f] = pack8(*reinterpret_cast<const v4u *>(r + fo[h][0]), *reinterpret_cast<const v4u *>(r + fo[h][1]));
        }
    };
    // One fragment (two 16-byte LDS reads) of K half h: index q < FN is row
    // operand block q, otherwise column operand block q - FN.
    auto read_frag = [&](v8i (&bf)[FN], v8i (&af)[FM], const uint8_t *slot, int h, int q) {
        const uint8_t *r = q < FN ? slot + b_frag + q * 32 * BK : slot + a_frag + (q - FN) * 32 * BK;
        const v8i v = pack8(*reinterpret_cast<const v4u *>(r + fo[h][0]), *reinterpret_cast<const v4u *>(r + fo[h][1]));
        if (q < FN) bf[q] = v;
        else af[q - FN] = v;
    };
    // This lane's scales of step kt: the A row it carries in each column
    // operand block, and the B block of this wave's rows (uniform).
    int scA[FM], scB = 127, nscA[FM], nscB = 127;
#pragma unroll
    for (int j = 0; j < FM; ++j) { scA[j] = 127; nscA[j] = 127; }
    auto read_scales = [&](int kt) {
        if (!BLK) return;
        const uint8_t *slot = smem + STAGES * SLOT + (kt % STAGES) * SCS;
#pragma unroll
        for (int j = 0; j < FM; ++j) nscA[j] = slot[wm * TM + j * 32 + lrow];
        nscB = slot[256 + 4 * ((wn * TN) / 128) + (kt & 3)];
    };
    // One K half of MFMAs with other work spread between them: the fragments
    // of the next half (read_slot / read_h) and, when refill_kt >= 0, the DMA
    // refill of a ring slot.  Issued in bursts, LDS reads and DMA instructions
    // stall the wave's in-order issue while their queues drain, and the MFMAs
    // queued behind them wait with them; spread out, they issue in the
    // shadow of the MFMAs.
    // With BF16 operands each tile takes two instructions per K half (one per
    // 16-byte part of its fragments); all tiles' first parts come before their
    // second parts, so consecutive instructions never chain on one accumulator.
    constexpr int NT = FN * FM;                    // accumulator tiles
    constexpr int NMF = NT * (BF ? 2 : 1);         // MFMA instructions per K half
    constexpr int NFR = FN + FM;                   // fragments per K half
    auto mma_mixed = [&](const v8i (&bf)[FN], const v8i (&af)[FM], v8i (&nb)[FN], v8i (&na)[FM],
                         const uint8_t *read_slot, int read_h, int refill_kt) {
#pragma unroll
        for (int t = 0; t < NMF; ++t) {
            const int i = (t % NT) / FM, j = (t % NT) % FM;
            if (BF) {
                if (t < NT) acc[i][j] = mfma32x32x16_bf16_part<0>(bf[i], af[j], acc[i][j]);
                else acc[i][j] = mfma32x32x16_bf16_part<1>(bf[i], af[j], acc[i][j]);
            } else if (BLK) {
                acc[i][j] = mfma32x32x64_s<FB, FA>(bf[i], af[j], acc[i][j], scB, scA[j]);
            } else {
                acc[i][j] = mfma32x32x64<FB, FA>(bf[i], af[j], acc[i][j]);
            }
            if (BLK && t == 0 && refill_kt >= 0) read_scales(refill_kt - STAGES + 1);
            // fragments of the next half: NFR reads spread over the NMF MFMAs
#pragma unroll
            for (int q = (t * NFR) / NMF; q < ((t + 1) * NFR) / NMF; ++q) read_frag(nb, na, read_slot, read_h, q);
            if (refill_kt >= 0) {
                if (t == 0) {
                    issue_scales(refill_kt);
                    if (UNI) set_step(refill_kt);
                }
#pragma unroll
                for (int q = (t * CPW) / NMF; q < ((t + 1) * CPW) / NMF; ++q) {
                    if (UNI) issue_fast(q);
                    else issue_one(refill_kt, q);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // ---- main loop ----
    // Slot kt % STAGES holds K step kt.  Fragment reads run one K half ahead
    // of the matrix cores (f0: first half, f1: second half), and the single
    // barrier per step sits between the halves: after it, step kt + 1 is in
    // LDS for everyone and nobody reads step kt's slot any more, so that slot
    // is refilled with step kt + STAGES while the second half computes.  The
    // scheduling barriers keep this order (left alone, the compiler reads
    // fragments just in time and exposes LDS latency before every few MFMAs).
    // Past the last step the DMA offsets are out of range: those loads deposit
    // zeros without touching memory and their slots are never read.
    static_assert(KH == 2, "the pipelined loop consumes two K halves per slot");
    v8i f0b[FN], f0a[FM], f1b[FN], f1a[FM];
#pragma unroll
    for (int s = 0; s < STAGES; ++s) issue(s);
    if (BLK && wave == 0) vmcnt_wait<(CPW + SCW) * (STAGES - 1)>();   // step 0 has landed
    else vmcnt_wait<CPW * (STAGES - 1)>();                            // (this wave's part)
    __syncthreads();
    read_frags(f0b, f0a, smem, 0);
    read_scales(0);
    for (int kt = 0; kt < nk; ++kt) {
        if (BLK) {
#pragma unroll
            for (int j = 0; j < FM; ++j) scA[j] = nscA[j];
            scB = nscB;
        }
        // Redefined each step so that the compiler forms the DMA offsets in
        // the loop instead of keeping one register per instruction live.
        if (!UNI) asm volatile("" : "+v"(doA0), "+v"(doA1), "+v"(doB0), "+v"(doB1), "+v"(dkc0), "+v"(dkc1));
        const uint8_t *cur = smem + (kt % STAGES) * SLOT;
        const uint8_t *nxt = smem + ((kt + 1) % STAGES) * SLOT;
        __builtin_amdgcn_sched_barrier(0);
        mma_mixed(f0b, f0a, f1b, f1a, cur, 1, -1);              // first half; reads the second
        if (BLK && wave == 0) vmcnt_wait<(CPW + SCW) * (STAGES - 2)>();
        else vmcnt_wait<CPW * (STAGES - 2)>();     // this wave's part of step kt + 1 has landed
        __syncthreads();                           // everyone's has; step kt's slot is no longer read
        mma_mixed(f1b, f1a, f0b, f0a, nxt, 0, kt + STAGES);     // second half; reads step kt + 1's
                                                                // first half, refills step kt's slot
    }
    vmcnt_wait<0>();                               // drain the (out-of-range) prefetches
    __syncthreads();                               // every wave's DMA has landed; the ring is free

    // ---- epilogue: scale, round to BF16, stage the tile in LDS, then write
    // whole row segments with 16-byte stores.
    // Accumulator register r of a 32x32 block holds row (of the first operand)
    // 8 * (r / 4) + 4 * (lane / 32) + r % 4 and column lane % 32, so lane l
    // holds four consecutive output columns n of output row m: an 8-byte
    // write.  Staged row m keeps its 16-byte chunks but stores chunk c at
    // c ^ (m % OCH), so the 32 rows one write instruction touches land on
    // different chunks, and a row read back is a permutation of one row.
#pragma unroll
    for (int j = 0; j < FM; ++j) {
        const uint32_t m = (uint32_t)(wm * TM + j * 32 + lrow);
#pragma unroll
        for (int i = 0; i < FN; ++i) {
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const uint32_t n = (uint32_t)(wn * TN + i * 32 + b * 8 + khalf * 4);
                const v16f &c = acc[i][j];
                const v2u v = pack_bf16x4(c[4 * b] * sc, c[4 * b + 1] * sc, c[4 * b + 2] * sc, c[4 * b + 3] * sc);
                const uint32_t chunk = (n >> 3) ^ (m % OCH);
                *reinterpret_cast<v2u *>(smem + m * (BN * 2) + chunk * 16 + (n & 4) * 2) = v;
            }
        }
    }
    __syncthreads();
    store_staged<BM, BN, THREADS, MODE>(p, smem, tid, spot, d_base, rowmask);
}

// ---------------------------------------------------------------------------
// Four-wave tiled kernel on the 16x16x128 instruction (FP8, dense form,
// per-tensor, per-channel or block scales).
// BM x BN output tile: 256 x 256; 128 x 256 where the 256-row tiles leave
// too many CUs idle; 256 x 224 or 256 x 192 where whole waves of those
// replace a partial wave of 256 x 256 tiles.  4 waves as 2 x 2, each owning
// BM/2 x BN/2 outputs as BN/32 weight blocks x BM/32 token blocks of 16 rows;
// a STAGES-slot direct-to-LDS ring of 128-byte K steps (2 slots of
// (256 + BN) x 128 bytes for BM = 256, 3 of 48 KB for BM = 128).  Against ring_kernel's 8 waves of 64 x 128 on 32x32x64 the
// 256-row form reads a third fewer LDS bytes per FLOP, and the
// 16x16x128 form draws less power per FLOP, so the chip, power-limited under
// this load, holds a higher clock.  One instruction spans the whole 128-byte
// K step: a fragment is a 16-row x 128-byte block, two 16-byte chunks per lane
// (row l % 16, chunks l / 16 and 4 + l / 16; A and B alike, so any K order
// inside the step is the same for both operands).
//
// LDS image: chunk c of ring row r is stored at c ^ ((r >> 1) & 7).  With it
// the lanes the LDS serves together in a fragment read hit distinct banks;
// ring_key, made for 32-row reads, leaves 2-way conflicts here (measured).
//
// Per K step kt, BN/32 x BM/32 MFMAs per wave in two halves (the first and the
// second half of the token blocks), each weight-block major:
//   - first half: the second half's token blocks of step kt are read in
//     between (their registers were freed by the last MFMAs of step kt - 1);
//   - before MFMA kBarAt: this wave's copies of step kt + 1 have landed
//     (vmcnt), then the step's one barrier: everyone's have, and every wave
//     has read all of step kt's fragments, so step kt's slot is free;
//   - MFMAs kDmaFrom .. kDmaTo - 1 carry the copies of step kt + STAGES into it;
//   - second half: each register set takes step kt + 1's fragment as soon as
//     its last use in step kt has issued.
// ---------------------------------------------------------------------------
template <int BM, int BN, int STAGES, int FA, int FB, int MODE, int SCL, bool KTAIL>
__global__ __launch_bounds__(256, 1) void tile16_kernel(GemmParams p) {
    constexpr bool CHN = SCL == SCALE_CHANNEL, BLK = SCL == SCALE_BLOCK;
    // The contiguous grouped form stays on ring_kernel: there, with every
    // expert's weights streaming from HBM, this kernel measured 4% slower
    // (1.90 against 1.82 ms on the 65536-row prefill).
    static_assert(FA != FMT_BF16 && FB != FMT_BF16 && (MODE == MODE_DENSE || (MODE == MODE_CONTIG && BM == 256 && BN == 256)),
                  "FP8 operands; dense form, or contiguous grouped with 256 x 256 tiles");
    constexpr int BK = 128, WM = 2, WN = 2, WAVES = WM * WN;
    constexpr int TM = BM / WM, TN = BN / WN;      // 128 (or 64) x 128 outputs per wave
    constexpr int FM = TM / 16, FN = TN / 16;      // token blocks, weight blocks
    constexpr int KCH = BK / 16, DROWS = 1024 / BK;
    constexpr int SLOT = (BM + BN) * BK;
    constexpr int CPA = BM / DROWS / WAVES;        // copy instructions per wave per step: A rows,
    constexpr int CPB = BN / DROWS / WAVES;        // B rows
    constexpr int CPW = CPA + CPB;
    constexpr int STAGE_OUT = BM * BN * 2;
    // Block scales (BLK): per ring slot, the step's E8M0 scale of each tile row
    // of A (bytes 0 .. BM-1, in A's row order) and the scale dword holding the
    // step's K block of each 128-row block of B (from byte 256).
    constexpr int SCS = BLK ? 512 : 0;
    constexpr int RING = STAGES * (SLOT + SCS);
    constexpr int MASK_AT = RING > STAGE_OUT ? RING : STAGE_OUT;   // contiguous form: the tile's row mask
    // per-channel form: the tile's row scales, channel scales and biases
    // (256 floats each), copied at the start, read by the epilogue
    constexpr int CH_AT = MASK_AT + (MODE == MODE_CONTIG ? BM / 8 : 0);
    constexpr int SMEM = CH_AT + (CHN ? 3 * 1024 : 0);
    constexpr int THREADS = 64 * WAVES;
    constexpr int OCH = BN / 8;
    constexpr int HALF = FN * FM / 2;              // MFMAs per half step
    // the step's one barrier, and the MFMAs that carry the copies
    // (256 x 256 dense tiles spread their copies up to MFMA 58: 0.3-0.5% faster
    // than up to 48 at 4096^3 and 8192 x 4096 x 4096 on one box, 1.0-1.5% on a
    // slower one, where up to 40 was 2.6% slower; the contiguous form, whose
    // weights come from HBM, keeps 48, having measured 0.7% slower at 58)
    constexpr int kBarAt = BM == 128 ? 10 : (BN == 192 ? 18 : 20), kDmaFrom = kBarAt,
                  kDmaTo = BM == 128 ? 28 : (BN == 192 ? 46 : (BN == 256 && MODE == MODE_DENSE ? 58 : 48));
    static_assert(((BM == 256 && (BN == 256 || BN == 224 || BN == 192)) || (BM == 128 && BN == 256)) &&
                      FN >= FM / 2 && CPA % 2 == 0, "shape");
    // block scales: each wave's weight rows must lie in one 128-row scale block
    static_assert(!BLK || BN == 256, "block scales: 256-column tiles");
    static_assert(STAGES >= 2 && RING <= 160 * 1024, "ring");
    static_assert(kBarAt >= 4 * (FM / 2 - 1) + 2 && kBarAt <= HALF && kDmaFrom >= kBarAt && kDmaTo <= 2 * HALF &&
                      kDmaTo - kDmaFrom >= CPW,
                  "schedule: the barrier after the first half's reads, before the second half's");

    __shared__ __attribute__((aligned(1024))) uint8_t smem[SMEM];

    // The contiguous grouped form computes up to two run-aligned tiles per
    // workgroup (place_contig_tile), one after the other; the dense form one.
    constexpr int PASSES = MODE == MODE_CONTIG ? 2 : 1;
    const int wave0 = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    ContigSlot cs{};
    if constexpr (MODE == MODE_CONTIG) {
        int tm, tn;
        tile_coords<true>(blockIdx.x, p.tiles_m, p.tiles_n, tm, tn);
        cs = contig_slot_tiles(p, lane_id_here(), tm);
    }
#pragma unroll 1
    for (int pass = 0; pass < PASSES; ++pass) {
    // With two passes the lane index is taken afresh in each (lane_id_here),
    // so that nothing derived from it (copy and fragment offsets) is hoisted
    // out of the loop and kept live next to the accumulators; threadIdx.x
    // itself would have to stay live since the kernel's start.
    const int tid = PASSES > 1 ? wave0 * 64 + lane_id_here() : (int)threadIdx.x;
    const int lane = tid & 63;
    const int wave = wave0;
    const int wm = wave % WM;
    const int wn = wave / WM;
    TileSpot spot;
    if constexpr (MODE == MODE_CONTIG) {
        if (!place_contig_tile(p, cs, pass, spot)) continue;   // uniform over the workgroup
    } else {
        if (!place_tile<BM, BN, MODE>(p, lane, spot)) return;
    }
    const int m0 = spot.m0, rows_m = spot.rows_m;
    const int n0 = spot.n0, rows_n = spot.rows_n;
    const int expert = spot.expert;
    uint64_t *const rowmask = reinterpret_cast<uint64_t *>(smem + MASK_AT);
    if constexpr (MODE == MODE_CONTIG) contig_row_mask<BM, WAVES>(p, spot, wave, lane, rowmask);
    const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t *)smem;
    const uint8_t *a_base = p.A + (int64_t)m0 * p.lda;
    const uint8_t *b_base = p.B + (int64_t)expert * p.b_gstride + (int64_t)n0 * p.ldb;
    const float sc = (CHN || BLK) ? 1.0f : p.scale_a[0] * p.scale_b[expert];
    // Rows past rows_m / rows_n fall outside the descriptors: zeros, no memory access.
    const v4i srdA = make_srd(a_base, rows_bytes(rows_m, p.lda));
    const v4i srdB = make_srd(b_base, rows_bytes(rows_n, p.ldb));

    // ---- copies.  Per step the tile is (BM + BN) / 8 copy instructions of 8
    // rows x 128 bytes, CPW per wave.  Copy qq of an operand fills its ring
    // rows 8 qq .. 8 qq + 7; lane l deposits row l / 8, stored chunk l % 8,
    // loading logical chunk (l % 8) ^ key(row).  The key of row 8 qq + r is
    // ((qq & 1) * 4 + (r >> 1)) & 7, so a lane's offset within the tile is
    // fixed per copy and kept in a register; each step only moves the
    // descriptor's base by the step's K offset (and shrinks its byte count by
    // as much, so rows past the tile's valid rows still read zeros), and past
    // the last step the byte count is 0.  The loop then spends one scalar
    // instruction per copy (the M0 address) and no vector ones.
    //   UNI (256-row tiles): waves 0-1 copy A's rows, waves 2-3 B's, copy i of
    //     wave w being copy w CPW + i of the tile; one descriptor per wave.
    //   otherwise (128-row tiles): wave w issues A's copies w CPA .. + CPA - 1
    //     and B's w CPB .. + CPB - 1 (measured 0.2-1.3% slower than UNI on the
    //     256-row tiles: one more descriptor to move per step).
    constexpr bool UNI = (BM / DROWS) % CPW == 0;
    auto key16 = [](uint32_t row) { return (row >> 1) & 7u; };
    const uint32_t lrow_in = (uint32_t)lane / KCH;
    const uint32_t dkc0 = (((uint32_t)lane % KCH) ^ key16(lrow_in)) * 16u;
    const uint32_t dkc1 = (((uint32_t)lane % KCH) ^ key16(DROWS + lrow_in)) * 16u;
    const int nk = (p.K + BK - 1) / BK;
    const bool wA = wave * CPW < BM / DROWS;       // UNI: this wave copies A (wave-uniform)
    // BLK: within each wave's TM rows, ring row 16 i + c holds tile row
    // FM c + i, so that token block i, column c is tile row FM c + i and a
    // lane's FM token-row scales are FM consecutive bytes (the fragment reads
    // are unchanged; only the rows the copies fetch move).
    auto a_row = [&](int s) { return BLK ? (s / TM) * TM + FM * (s % 16) + (s % TM) / 16 : s; };
    uint32_t lo_q[CPW];                            // UNI: this wave's copies; else A's, then B's
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
        const bool isA = UNI ? wA : i < CPA;
        const int qq = UNI ? (wave * CPW + i) % (BM / DROWS) : (isA ? wave * CPA + i : wave * CPB + (i - CPA));
        const int row = qq * DROWS + (int)lrow_in;
        lo_q[i] = (uint32_t)(isA ? a_row(row) : row) * (uint32_t)(isA ? p.lda : p.ldb) + ((qq & 1) ? dkc1 : dkc0);
    }
    const v4i srd0A = UNI ? (wA ? srdA : srdB) : srdA;
    const uint64_t baseA = ((uint64_t)(uint32_t)srd0A[1] << 32) | (uint32_t)srd0A[0];
    const uint64_t baseB = ((uint64_t)(uint32_t)srdB[1] << 32) | (uint32_t)srdB[0];
    const uint32_t lds_wa = lds0 + (uint32_t)(wave * (UNI ? CPW : CPA)) * 1024u;
    const uint32_t lds_wb = lds0 + (uint32_t)(BM / DROWS + wave * CPB) * 1024u;
    v4i srdAk = srd0A, srdBk = srdB;
    uint32_t lds_a = 0, lds_b = 0;
    // K tail (K not a multiple of 128): on the last step, lanes whose chunk
    // starts at or past K add kOobOffset (their offset, below 2^31 before,
    // then lies in [2^31, 2^32): past every descriptor).  The lane's chunk
    // depends on the key parity of its copy's row group qq.  CPA is even, and
    // so is CPW where UNI holds, so for A's copies (and all of UNI's) that is
    // the parity of i; B's copy i is qq = wave CPB + i - CPA, whose parity
    // for odd CPB (224-column tiles) also flips with the wave's.
    constexpr bool FLIPB = !UNI && (CPB & 1);
    const bool flipb = FLIPB && (wave & 1);
    uint32_t ko0 = 0, ko1 = 0, kob0 = 0, kob1 = 0;
    auto set_step = [&](int kd) {                  // the copies of step kd follow
        const uint64_t ba = baseA + (uint64_t)kd * BK;
        srdAk[0] = (int)(uint32_t)ba;
        srdAk[1] = (int)(uint32_t)(ba >> 32);
        srdAk[2] = kd < nk ? srd0A[2] - kd * BK : 0;
        lds_a = lds_wa + (uint32_t)(kd % STAGES) * SLOT;
        if (!UNI) {
            const uint64_t bb = baseB + (uint64_t)kd * BK;
            srdBk[0] = (int)(uint32_t)bb;
            srdBk[1] = (int)(uint32_t)(bb >> 32);
            srdBk[2] = kd < nk ? srdB[2] - kd * BK : 0;
            lds_b = lds_wb + (uint32_t)(kd % STAGES) * SLOT;
        }
        if (KTAIL) {
            const int lim = p.K - kd * BK;
            ko0 = (int)dkc0 < lim ? 0u : kOobOffset;
            ko1 = (int)dkc1 < lim ? 0u : kOobOffset;
            kob0 = flipb ? ko1 : ko0;
            kob1 = flipb ? ko0 : ko1;
        }
    };
    auto issue_one = [&](int i) {
        const bool inB = FLIPB && i >= CPA;
        const uint32_t voff = KTAIL ? lo_q[i] + ((i & 1) ? (inB ? kob1 : ko1) : (inB ? kob0 : ko0)) : lo_q[i];
        if (UNI || i < CPA) dma16_m0(srdAk, voff, lds_a + (uint32_t)i * 1024u);
        else dma16_m0(srdBk, voff, lds_b + (uint32_t)(i - CPA) * 1024u);
    };
    // BLK: every wave copies step kd's scales into the scale slot of its ring
    // slot: A's BM row scales (4 per lane) and B's scale dwords (one per
    // 128-row block, the dword holding K block kd).  The four waves write the
    // same bytes; leaving it to one wave put a branch in the loop, across
    // which the compiler moved the first half's MFMAs behind the barrier.
    // Rows past the scale array (or steps past the last) read zeros; bytes of
    // rows past M only reach outputs that are not written.
    const int64_t sa_bytes = (int64_t)((p.K + 127) / 128) * p.lds_sa;
    const int64_t sb_bytes = (int64_t)((p.N + 127) / 128) * p.lds_sb;
    // (contiguous form: token-row scales by global row, weight-block scales of the tile's expert)
    const v4i srdSA = BLK ? make_srd(p.sfa, (uint32_t)sa_bytes) : v4i{0, 0, 0, 0};
    const v4i srdSB = BLK ? make_srd(p.sfb + (int64_t)expert * sb_bytes, (uint32_t)sb_bytes) : v4i{0, 0, 0, 0};
    const uint32_t scl_base = lds0 + STAGES * SLOT;
    constexpr int SCW = BLK ? 2 : 0;               // scale copies per wave per step
    auto issue_scales = [&](int kd) {
        if (!BLK) return;
        const uint32_t slot = scl_base + (uint32_t)(kd % STAGES) * SCS;
        const bool ka = kd < nk && 4 * lane < BM;
        dma4(srdSA, ka ? (uint32_t)(kd * p.lds_sa + m0 + 4 * lane) : kOobOffset, slot);
        const bool kb = kd < nk && lane < BN / 128;
        dma4(srdSB, kb ? (uint32_t)((n0 / 128 + lane) * p.lds_sb + (kd & ~3)) : kOobOffset, slot + 256);
    };

    // ---- fragments (blocks start at multiples of 16 rows, so the key of a
    // lane's row depends on l % 16 only)
    const int r16 = lane & 15;
    const int kg = lane >> 4;
    const uint32_t key = key16((uint32_t)r16);
    const uint32_t fo0 = (uint32_t)r16 * BK + (((uint32_t)kg ^ key) & 7u) * 16u;
    const uint32_t fo1 = (uint32_t)r16 * BK + (((uint32_t)(4 + kg) ^ key) & 7u) * 16u;
    const uint32_t a_frag = (uint32_t)(wm * TM) * BK;
    const uint32_t b_frag = (uint32_t)BM * BK + (uint32_t)(wn * TN) * BK;
    auto frag = [&](const uint8_t *slot, uint32_t base, int blk) {
        const uint8_t *r = slot + base + blk * 16 * BK;
        return pack8(*reinterpret_cast<const v4u *>(r + fo0), *reinterpret_cast<const v4u *>(r + fo1));
    };

    v4f acc[FN][FM];
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int i = 0; i < FM; ++i) acc[j][i] = (v4f){0, 0, 0, 0};
    v8i wf[FN], tf[FM];                            // one register set per block, reused in place

    // BLK: this lane's token-row scales of a step, FM bytes (rows FM c + i,
    // c = l % 16), and the wave's weight-block scale; read one step ahead.
    uint32_t sa_lo = 0, sa_hi = 0, nsa_lo = 0, nsa_hi = 0;
    int scb = 0, nscb = 0;
    auto read_scales = [&](int kt) {
        if (!BLK) return;
        const uint8_t *slot = smem + STAGES * SLOT + (kt % STAGES) * SCS;
        const uint8_t *ra = slot + wm * TM + FM * r16;
        if (FM == 8) {
            const v2u v = *reinterpret_cast<const v2u *>(ra);
            nsa_lo = v[0];
            nsa_hi = v[1];
        } else {
            nsa_lo = *reinterpret_cast<const uint32_t *>(ra);
        }
        nscb = slot[256 + 4 * wn + (kt & 3)];
    };

    auto step = [&](int kt) {
        const uint8_t *cur = smem + (kt % STAGES) * SLOT;
        const uint8_t *nxt = smem + ((kt + 1) % STAGES) * SLOT;
        if (BLK) {
            sa_lo = nsa_lo;
            sa_hi = nsa_hi;
            scb = nscb;
        }
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int ii = 0; ii < FM / 2; ++ii) {
                    const int i = h * (FM / 2) + ii;
                    const int t = h * HALF + j * (FM / 2) + ii;
                    if (t == kBarAt) {
                        // this wave's copies of step kt + 1 have landed
                        vmcnt_wait<(CPW + SCW) * (STAGES - 2)>();
                        __syncthreads();           // everyone's have; step kt's slot is no longer read
                    }
                    if (BLK)                       // token block i's scale: byte i % 4 of its word
                        acc[j][i] = mfma16x16x128_sb<FB, FA>(wf[j], tf[i], acc[j][i], scb, (int)(i < 4 ? sa_lo : sa_hi), i);
                    else acc[j][i] = mfma16x16x128<FB, FA>(wf[j], tf[i], acc[j][i]);
                    if (BLK && t == kBarAt) read_scales(kt + 1);
                    if (h == 0) {
                        if (t % 4 == 1 && t / 4 < FM / 2) tf[FM / 2 + t / 4] = frag(cur, a_frag, FM / 2 + t / 4);
                    } else {
                        if (j < FM / 2 && ii == 1) tf[j] = frag(nxt, a_frag, j);
                        if (ii == FM / 2 - 1) wf[j] = frag(nxt, b_frag, j);
                    }
                    if (t == kDmaFrom) {
                        set_step(kt + STAGES);
                        issue_scales(kt + STAGES);
                    }
                    if (t >= kDmaFrom && t < kDmaTo) {
                        constexpr int SPAN = kDmaTo - kDmaFrom;
                        const int u = t - kDmaFrom;
#pragma unroll
                        for (int q = (u * CPW) / SPAN; q < ((u + 1) * CPW) / SPAN; ++q) issue_one(q);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
    };

    // Per-channel form: wave w copies rows (and channels) 64 w .. 64 w + 63 of
    // the tile's row scales, channel scales and biases into LDS, one dword per
    // lane, before its ring copies, so the wait for step 0 covers them.
    // Entries past M or N (and absent arrays) read as zeros; the epilogue then
    // reads them from LDS instead of waiting on global loads per weight block
    // at the end of the kernel.
    if constexpr (CHN) {
        // an absent array of scales is written as ones instead (an absent
        // bias reads zeros through an empty descriptor)
        const uint32_t ch_lds = lds0 + (uint32_t)CH_AT + (uint32_t)wave * 256u;
        const uint32_t voff = 4u * (uint32_t)(wave * 64 + lane);
        float *const ch = reinterpret_cast<float *>(smem + CH_AT) + wave * 64 + lane;
        if (p.ch_sa) dma4(make_srd(p.ch_sa + m0, rows_bytes(rows_m, 4)), voff, ch_lds);
        else ch[0] = 1.0f;
        if (p.ch_sb) dma4(make_srd(p.ch_sb + n0, rows_bytes(rows_n, 4)), voff, ch_lds + 1024u);
        else ch[256] = 1.0f;
        dma4(p.bias ? make_srd(p.bias + n0, rows_bytes(rows_n, 4)) : make_srd(p.A, 0u), voff, ch_lds + 2048u);
    }

    // ---- main loop (past the last step the copy offsets are out of range:
    // zeros, no memory access, never read).  With STAGES slots the copies of
    // step kt + STAGES refill step kt's slot, so STAGES - 1 steps of copies are
    // in flight.
#pragma unroll
    for (int st = 0; st < STAGES; ++st) {
        set_step(st);
        issue_scales(st);
#pragma unroll
        for (int i = 0; i < CPW; ++i) issue_one(i);
    }
    // this wave's part of step 0 has landed
    vmcnt_wait<(CPW + SCW) * (STAGES - 1)>();
    __syncthreads();
    read_scales(0);
#pragma unroll
    for (int j = 0; j < FN; ++j) wf[j] = frag(smem, b_frag, j);
#pragma unroll
    for (int i = 0; i < FM / 2; ++i) tf[i] = frag(smem, a_frag, i);
    // Nothing outstanding on the LDS / scalar-load counter at the loop head:
    // otherwise the compiler assumes a scalar load may still be in flight
    // there and waits for every LDS read (lgkmcnt(0)) at the top of each step.
    lgkmcnt_wait<0>();
    for (int kt = 0; kt < nk; ++kt) step(kt);
    vmcnt_wait<0>();                               // drain the (out-of-range) prefetches
    __syncthreads();                               // every wave's copies have landed; the ring is free
    __builtin_amdgcn_sched_barrier(0);

    // ---- epilogue: accumulator register r of a 16x16 block holds weight row
    // 4 (l / 16) + r and token column l % 16, so a lane holds four consecutive
    // output columns of one output row: scale, round to BF16, stage in LDS as
    // ring_kernel does, then 16-byte stores of whole row segments.  (The lane
    // index is taken afresh here so that no lane value stays live across the
    // loop next to the accumulators.)
    const int el = PASSES > 1 ? lane_id_here() : (int)__lane_id();
    const int er16 = el & 15, ekg = el >> 4;
    auto put = [&](int i, int j, v2u v) {
        const uint32_t m = (uint32_t)(wm * TM + i * 16 + er16);
        const uint32_t n = (uint32_t)(wn * TN + j * 16 + ekg * 4);
        const uint32_t chunk = stage_chunk<OCH>(n >> 3, m);
        *reinterpret_cast<v2u *>(smem + m * (BN * 2) + chunk * 16 + (n & 4) * 2) = v;
    };
    // The loop orders below are the ones that keep the compiler's copies of
    // the 256 accumulators out of AGPRs within the register budget (the other
    // order spills in each case).
    if constexpr (CHN) {
        // per token block, the row scale of this lane's row, then per weight
        // block the four channels' scales and biases, read from the copies in
        // LDS where they are used (the other loop order, and keeping a weight
        // block's terms in registers across the token blocks, spill).  Against
        // global loads per weight block here: 4096^3 0.3-0.8 us faster (of
        // ~51), four interleaved pairs on one box.
        const float *ch = reinterpret_cast<const float *>(smem + CH_AT);
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const float sa = ch[wm * TM + i * 16 + er16];
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int c0 = wn * TN + j * 16 + ekg * 4;
                const v4f sv = *reinterpret_cast<const v4f *>(ch + 256 + c0);
                const v4f bv = *reinterpret_cast<const v4f *>(ch + 512 + c0);
                const v4f &c = acc[j][i];
                put(i, j, pack_bf16x4(c[0] * sa * sv[0] + bv[0], c[1] * sa * sv[1] + bv[1],
                                      c[2] * sa * sv[2] + bv[2], c[3] * sa * sv[3] + bv[3]));
            }
            __builtin_amdgcn_sched_barrier(0);     // one token block at a time: bounded live registers
        }
    } else if constexpr (!BLK) {
#pragma unroll
        for (int i = 0; i < FM; ++i) {
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const v4f &c = acc[j][i];
                put(i, j, pack_bf16x4(c[0] * sc, c[1] * sc, c[2] * sc, c[3] * sc));
            }
            __builtin_amdgcn_sched_barrier(0);     // one token block at a time: bounded live registers
        }
    }
    if constexpr (!BLK) {
        __syncthreads();
        const int etid = PASSES > 1 ? wave * 64 + el : tid;   // formed afresh, as above
        store_staged<BM, BN, THREADS, MODE>(p, smem, etid, spot, p.D, rowmask);
    } else {
        // Block scales: each wave stages its own TM x TN outputs in a private
        // part of the (now free) ring, in its token-block order (row r =
        // 16 i + c at r * TN * 2 bytes, chunk at stage_chunk<WCH>(c, r)), and
        // stores each token block's 16 rows as soon as they are staged: the
        // stores of one block overlap the staging of the next, and no
        // workgroup barrier is needed (a wave's LDS accesses complete in
        // order).  Staged in tile-row order, the permuted rows (FM c + i)
        // were 4096^3 55.1-55.9 us against 51.3-52.1 this way; the other
        // forms measured 0-3% slower with these half-width row segments.
        constexpr int WCH = TN / 8;                // 16-byte chunks per row of the wave's block
        constexpr int WROW = TN * 2;
        static_assert(WAVES * TM * WROW <= SMEM, "per-wave staging fits the ring");
        uint8_t *const ws = smem + wave * (TM * WROW);
        const int ncol0 = n0 + wn * TN;
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const uint32_t r = (uint32_t)(i * 16 + er16);
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const v4f &c = acc[j][i];
                const uint32_t n = (uint32_t)(j * 16 + ekg * 4);
                *reinterpret_cast<v2u *>(ws + r * WROW + stage_chunk<WCH>(n >> 3, r) * 16 + (n & 4) * 2) =
                    pack_bf16x4(c[0] * sc, c[1] * sc, c[2] * sc, c[3] * sc);
            }
            __builtin_amdgcn_sched_barrier(0);     // staged before read back
#pragma unroll
            for (int q = el; q < 16 * WCH; q += 64) {
                const int rr = q / WCH, cc = q % WCH;
                const uint32_t wr = (uint32_t)(i * 16 + rr);
                const v4u v = *reinterpret_cast<const v4u *>(ws + wr * WROW + stage_chunk<WCH>(cc, wr) * 16);
                const int m = wm * TM + FM * rr + i;   // token block i, column rr
                const int n = ncol0 + cc * 8;
                if (m < rows_m && (MODE != MODE_CONTIG || row_in_mask(rowmask, m)))
                    store_chunk<MODE>(p.D + (int64_t)(m0 + m) * p.ldd + n, v, p.N - n);
            }
            __builtin_amdgcn_sched_barrier(0);     // one token block at a time: bounded live registers
        }
    }
    if (PASSES > 1) __syncthreads();               // the staged tile is read out before the ring refills
    }
}

// ---------------------------------------------------------------------------
// Streaming swap-AB kernel.
// 4 waves; wave w streams weight rows [n0 + w*WR, +WR) (WR = 128, or 64 when
// there are too few groups to fill the CUs or the token blocks are many) as
// WR/16 row blocks of the 16x16x128 instruction.  Tokens: CB blocks of 16
// per pass over the weights, CB in {1, 2, 4} for few tokens and {8, 12} for
// up to 128 / 192 (with WR = 64, so that the WR/16 x CB accumulators fit).  Every weight byte is used by exactly one wave; it
// still passes through the wave's own LDS ring, because copying whole lines
// there and reading the operand layout back beats loading that layout
// directly (see the weight-copy comment below).  Tokens form up to CB column
// blocks of 16; their tile is shared by the 4 waves, so it is copied once per
// workgroup into a small LDS ring and read from there.  DEPTH ring slots keep
// DEPTH-1 K blocks of copies in flight per wave.
// ---------------------------------------------------------------------------
template <int WR, int CB, int FA, int FB, int DEPTH, int MODE, int SCL>
__global__ __launch_bounds__(256, 1) void swap_kernel(GemmParams p) {
    constexpr bool BLK = SCL == SCALE_BLOCK;
    // with block scales each wave's rows (WR of them, starting at a multiple of
    // WR) must lie in one 128-row scale block
    static_assert(!BLK || WR == 128 || WR == 64, "block scales: each wave's rows within one 128-row scale block");
    constexpr int RB = WR / 16;
    constexpr int ROWB = 128;                      // K bytes per pipeline stage
    constexpr int TR = CB <= 2 ? 32 : 16 * CB;     // token rows staged per stage (>= 32: one DMA per wave)
    constexpr int TDMA = TR / 32;                  // token DMA instructions per wave per stage (8 rows each)
    // 12 token blocks (up to 192 tokens): each step's 48 MFMAs per wave take
    // about as long as a weight copy from HBM, so the weights get two steps in
    // flight (DW = 3 slots per wave) and the tokens, L2 hits, one: both copies
    // of a step are issued after its barrier, tokens first, which lets 2 token
    // slots do (no wave still reads the slot being refilled) and lets the wait
    // before a step leave the newest weight copies in flight.  Measured with
    // 16 groups of 160 tokens: 121.5 -> 115.3 us at 4096 x 7168, 71.7 -> 65.4
    // us at 7168 x 2048; with 8 blocks (96 tokens) -1% and +2%, so those keep
    // the 2-step ring.
    constexpr bool DEEPW = CB >= 12;
    constexpr int DW = DEEPW ? 3 : DEPTH;          // weight ring slots per wave
    constexpr int TS = DEEPW ? 2 : DEPTH + 1;      // token ring slots
    constexpr int TSLOT = TR * ROWB;
    constexpr int WLOADS = RB * 2 + (BLK ? 1 : 0); // weight loads (and the block scale) per wave per stage
    constexpr int SDMA = BLK ? 1 : 0;              // token-scale DMA of wave 0 per stage
    constexpr int SCS = BLK ? 256 : 0;             // token-scale bytes per ring slot
    constexpr int WSLOT = WR * ROWB;               // one stage of one wave's weight rows
    constexpr int WRING = 4 * DW * WSLOT;          // the four waves' weight rings
    constexpr int WSC = BLK ? 256 : 0;             // one stage of one wave's weight-scale copy
    constexpr int WSC_OFF = WRING + TS * TSLOT + TS * SCS;
    static_assert(RB >= 1 && CB >= 1 && DEPTH >= 2, "shape");
    static_assert((DEPTH - 1) * (WLOADS + TDMA + SDMA) < 64 && 2 * WLOADS + TDMA + SDMA < 64, "loads in flight");
    static_assert(WSC_OFF + 4 * DW * WSC <= 160 * 1024, "LDS");

    // [weight rings of the 4 waves | token ring | token-scale ring | weight-scale slots]
    __shared__ __attribute__((aligned(1024))) uint8_t smem[WSC_OFF + 4 * DW * WSC];
    uint8_t *const tsm = smem + WRING;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = (MODE == MODE_MASKED) ? (int)(blockIdx.x / p.tiles_n) : 0;
    const int nb = (MODE == MODE_MASKED) ? (int)(blockIdx.x % p.tiles_n) : (int)blockIdx.x;

    // Valid token count: read on the device, clamped; an empty group exits
    // before forming any address ("MLS three memory-access bugs", Bug 2: a
    // fully masked tile must not issue loads).  The exit is uniform over the
    // workgroup.
    const int mg = (MODE == MODE_MASKED) ? min(max(p.masked_m[g], 0), p.cap) : p.M;
    if (mg <= 0) return;
    const int nw = nb * 4 * WR + wave * WR;        // first weight row of this wave
    const int rows_w = max(0, min(p.N - nw, WR));  // may be 0 on the N tail: the wave then loads
                                                   // nothing but still takes part in the barriers

    const uint8_t *w_base = p.B + (int64_t)g * p.b_gstride + (int64_t)min(nw, p.N) * p.ldb;
    const uint8_t *t_base = p.A + (int64_t)g * p.a_gstride;
    uint16_t *d_base = p.D + (int64_t)g * p.d_gstride;
    const float sc = BLK ? 1.0f : p.scale_a[0] * p.scale_b[g];
    const v4i srdW = make_srd(w_base, rows_bytes(rows_w, p.ldb));
    // Block scales of group g: token rows [kb][lds_sa], weight blocks [nb][lds_sb];
    // this wave's 128 weight rows are one scale block.
    const int nk_ = (p.K + 127) / 128;
    const uint8_t *sa_g = BLK ? p.sfa + (int64_t)g * nk_ * p.lds_sa : p.A;
    const uint8_t *sb_g = BLK ? p.sfb + (int64_t)g * ((p.N + 127) / 128) * p.lds_sb : p.A;
    const v4i srdSB = BLK ? make_srd(sb_g, (uint32_t)(((p.N + 127) / 128) * p.lds_sb)) : v4i{0, 0, 0, 0};
    const uint32_t sb_row = BLK ? (uint32_t)(min(nw, p.N) / 128) * (uint32_t)p.lds_sb : 0u;
    const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t *)tsm;
    const uint32_t wlds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t *)smem +
                          (uint32_t)wave * (DW * WSLOT);

    // Operand layout used for both operands of v_mfma 16x16x128: lane l
    // carries row (l & 15) and, of each 128-byte K block, the bytes
    // [(l >> 4) * 16, +16) and [64 + (l >> 4) * 16, +16).  Loaded straight
    // from memory that layout puts consecutive lanes on 16 different rows, and
    // each load instruction becomes 64 separate 16-byte accesses; copied
    // through LDS with 8 lanes per 128-byte line, the same weight stream ran
    // 3.5% faster (measured with the masked decode workload).  So each wave
    // copies its 128 rows of a K step into its own LDS slot: instruction
    // 2 r + h fills rows 16 r + 8 h .. +8, lane l taking row 16 r + 8 h + l / 8
    // and storing logical chunk (l % 8) ^ key(row) at position l % 8, with
    // key(row) = (row >> 1) & 7, so that the 16 rows of one chunk that a
    // fragment read touches sit on 16 different bank groups.
    const int r16 = lane & 15;
    const int kg = lane >> 4;
    const uint32_t wrow = (uint32_t)lane >> 3;
    const uint32_t wch0 = (((uint32_t)lane & 7u) ^ ((wrow >> 1) & 7u)) * 16u;          // rows 0..7 of a block
    const uint32_t wch1 = (((uint32_t)lane & 7u) ^ (((wrow + 8u) >> 1) & 7u)) * 16u;   // rows 8..15
    const uint32_t wo0 = wrow * (uint32_t)p.ldb + wch0, wo1 = (wrow + 8u) * (uint32_t)p.ldb + wch1;
    const uint32_t wkey = ((uint32_t)r16 >> 1) & 7u;
    const uint32_t wf0 = (uint32_t)r16 * ROWB + (((uint32_t)kg ^ wkey) * 16u);
    const uint32_t wf1 = (uint32_t)r16 * ROWB + (((uint32_t)(4 + kg) ^ wkey) * 16u);

    // Token DMA: instruction i of this wave covers staged rows
    // (wave * TDMA + i) * 8 .. +8; lane l deposits row l / 8, stored chunk
    // l % 8, loading logical chunk (l % 8) ^ key(row) with the weights' key
    // (row >> 1) & 7, under which the fragment reads of any 16 rows are free of
    // bank conflicts.
    uint32_t t_dma_off[TDMA];
    uint32_t t_dma_kc[TDMA];
#pragma unroll
    for (int i = 0; i < TDMA; ++i) {
        const int row = (wave * TDMA + i) * 8 + (lane >> 3);
        const uint32_t c = ((uint32_t)(lane & 7) ^ (((uint32_t)row >> 1) & 7u)) & 7u;
        t_dma_kc[i] = c * 16;
        t_dma_off[i] = (uint32_t)((int64_t)row * p.lda) + c * 16;
    }
    // Token fragment reads: block c, row c*16 + r16, logical chunks kg, 4 + kg.
    uint32_t t_frag[CB][2];
#pragma unroll
    for (int c = 0; c < CB; ++c) {
        const uint32_t row = (uint32_t)(c * 16 + r16);
        const uint32_t key = (row >> 1) & 7u;
        t_frag[c][0] = row * ROWB + ((((uint32_t)kg) ^ key) & 7u) * 16u;
        t_frag[c][1] = row * ROWB + ((((uint32_t)kg + 4u) ^ key) & 7u) * 16u;
    }

    const int nk = (p.K + ROWB - 1) / ROWB;

    for (int t0 = 0; t0 < mg; t0 += CB * 16) {
        const int mt = min(mg - t0, CB * 16);
        // Token rows past the valid count fall outside this descriptor: the DMA
        // deposits zeros for them and never fetches them (the NaN-filled rows
        // behind them never reach the matrix cores: same page, Bug 3).
        const v4i srdT = make_srd(t_base + (int64_t)t0 * p.lda, rows_bytes(mt, p.lda));
        // Token-row scales of this token block (wave 0): rows past the group's
        // count may read other in-range bytes, which reach only unwritten rows.
        const v4i srdST = BLK ? make_srd(sa_g, (uint32_t)(nk_ * p.lds_sa)) : v4i{0, 0, 0, 0};
        __syncthreads();                           // the ring is free (previous token block done)

        v4f acc[RB][CB];
#pragma unroll
        for (int r = 0; r < RB; ++r)
#pragma unroll
            for (int c = 0; c < CB; ++c) acc[r][c] = (v4f){0, 0, 0, 0};


        // One stage: this wave's weight copies (into its own slot), then its
        // token DMA.  Past the last K block every offset is out of range: no
        // memory traffic, zeros, and the stage is never consumed.
        auto load_w = [&](int slot, int kt) {
            const uint32_t k0 = (uint32_t)kt * ROWB;
            const bool in0 = (kt < nk) && (int)(k0 + wch0) < p.K;
            const bool in1 = (kt < nk) && (int)(k0 + wch1) < p.K;
#pragma unroll
            for (int r = 0; r < RB; ++r) {
                const uint32_t roff = (uint32_t)(r * 16) * (uint32_t)p.ldb + k0;
                const uint32_t dst = wlds + (uint32_t)(slot * WSLOT + r * 2048);
                dma16(srdW, in0 ? wo0 + roff : kOobOffset, dst);
                dma16(srdW, in1 ? wo1 + roff : kOobOffset, dst + 1024u);
            }
            // this wave's weight-block scale of step kt: the dword holding it, into
            // the wave's own slot (copied, not loaded into a register, so that every
            // load of the stage is counted by the waits below)
            if (BLK)
                dma4(srdSB, kt < nk && lane == 0 ? sb_row + ((uint32_t)kt & ~3u) : kOobOffset,
                     lds0 - (uint32_t)WRING + (uint32_t)(WSC_OFF + (wave * DW + slot) * WSC));
        };
        auto load_t = [&](int kt) {
            const uint32_t k0 = (uint32_t)kt * ROWB;
#pragma unroll
            for (int i = 0; i < TDMA; ++i) {
                const bool in = (kt < nk) && (int)(k0 + t_dma_kc[i]) < p.K;
                dma16(srdT, in ? t_dma_off[i] + k0 : kOobOffset,
                      lds0 + (uint32_t)((kt % TS) * TSLOT) + (uint32_t)(wave * TDMA + i) * 1024u);
            }
            if (BLK && wave == 0) {
                const bool in = (kt < nk) && 4 * lane < CB * 16;
                dma4(srdST, in ? (uint32_t)kt * (uint32_t)p.lds_sa + (uint32_t)(t0 + 4 * lane) : kOobOffset,
                     lds0 + (uint32_t)(TS * TSLOT) + (uint32_t)((kt % TS) * SCS));
            }
        };
        auto load = [&](int slot, int kt) {
            load_w(slot, kt);
            load_t(kt);
        };
        // Step kt's MFMAs: token fragments of token slot kt % TS, weight
        // fragments of this wave's weight slot `wslot`.
        auto compute = [&](int kt, int wslot) {
            const uint8_t *ts = tsm + (kt % TS) * TSLOT;
            v8i tf[CB];
            int tsc[CB];
#pragma unroll
            for (int c = 0; c < CB; ++c) {
                tf[c] = pack8(*reinterpret_cast<const v4u *>(ts + t_frag[c][0]),
                              *reinterpret_cast<const v4u *>(ts + t_frag[c][1]));
                tsc[c] = BLK ? (int)tsm[TS * TSLOT + (kt % TS) * SCS + c * 16 + r16] : 127;
            }
            const uint8_t *ws = smem + wave * (DW * WSLOT) + wslot * WSLOT;
            const int wsc = BLK ? (int)smem[WSC_OFF + (wave * DW + wslot) * WSC + (kt & 3)] : 127;
#pragma unroll
            for (int r = 0; r < RB; ++r) {
                const v8i wf = pack8(*reinterpret_cast<const v4u *>(ws + r * 2048 + wf0),
                                     *reinterpret_cast<const v4u *>(ws + r * 2048 + wf1));
#pragma unroll
                for (int c = 0; c < CB; ++c) {
                    if (BLK) acc[r][c] = mfma16x16x128_s<FB, FA>(wf, tf[c], acc[r][c], wsc, tsc[c]);
                    else acc[r][c] = mfma16x16x128<FB, FA>(wf, tf[c], acc[r][c]);
                }
            }
        };

        if constexpr (DEEPW) {
            // Copies in issue order: T0 W0 W1 | T1 W2 | T2 W3 | ... (Tk: step
            // k's tokens, Wk: this wave's weights of step k, the group after
            // "|" issued in step k - 1 after its barrier).  Before step kt only
            // W(kt + 1) may still be in flight; T(kt + 1) refills the token slot
            // of step kt - 1, which every wave has read before the barrier, and
            // W(kt + 2) this wave's weight slot of step kt - 1.
            load_t(0);
            load_w(0, 0);
            load_w(1, 1);
            __builtin_amdgcn_sched_barrier(0);
            for (int kt = 0; kt < nk; ++kt) {
                vmcnt_wait<WLOADS>();              // every copy of step kt has landed
                __syncthreads();                   // every wave's, and step kt - 1 is read
                load_t(kt + 1);
                load_w((kt + 2) % DW, kt + 2);
                __builtin_amdgcn_sched_barrier(0);
                compute(kt, kt % DW);
                __builtin_amdgcn_sched_barrier(0);
            }
        } else {
            // Software pipeline over K blocks, branch-free: the scheduling
            // barriers keep the load groups in slot order, so every wait is exact.
#pragma unroll
            for (int s = 0; s < DEPTH - 1; ++s) {
                load(s, s);
                __builtin_amdgcn_sched_barrier(0);
            }
            for (int kb = 0; kb < nk; kb += DEPTH) {
#pragma unroll
                for (int s = 0; s < DEPTH; ++s) {
                    const int kt = kb + s;
                    load((s + DEPTH - 1) % DEPTH, kt + DEPTH - 1);
                    __builtin_amdgcn_sched_barrier(0);
                    // every load of step kt (older than the DEPTH - 1 newer stages) has landed
                    if (BLK && wave == 0) vmcnt_wait<(DEPTH - 1) * (WLOADS + TDMA + SDMA)>();
                    else vmcnt_wait<(DEPTH - 1) * (WLOADS + TDMA)>();
                    __syncthreads();               // every wave's token DMA of step kt has landed
                    compute(kt, s);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
        vmcnt_wait<0>();                           // drain the out-of-range prefetches

        // Epilogue: accumulator register q of a 16x16 block holds weight row
        // 4 * (lane / 16) + q and token column lane % 16.
#pragma unroll
        for (int c = 0; c < CB; ++c) {
            const int tok = t0 + c * 16 + r16;
            if (tok >= mg) continue;
            uint16_t *drow = d_base + (int64_t)tok * p.ldd;
#pragma unroll
            for (int r = 0; r < RB; ++r) {
                const int n = nw + r * 16 + kg * 4;
                const v4f &a = acc[r][c];
                const v2u v = pack_bf16x4(a[0] * sc, a[1] * sc, a[2] * sc, a[3] * sc);
                store_bf16x4(drow, n, p.N - n, v);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Decode kernel: the dense form with few tokens (M <= 64), swap-AB: weights on
// the instruction's 16-row side, tokens in CB column blocks of 16 (section 1.1
// of "One transpose, half the compute": with few tokens the work is bound by
// weight bandwidth).  The 16x16x128 operand layout puts lane l on row l % 16, so loading
// it straight from memory puts consecutive lanes on 16 different rows and
// splits every 1 KB load instruction into 64 separate 16-byte accesses in the
// vector memory pipeline (measured at M = 64, N = 4096, K = 7168: the token
// loads alone took 16 of the 21 us, and 8.6 us with the same bytes read by
// consecutive lanes).  Here each wave copies its K steps into its own LDS ring
// with direct-to-LDS loads in which every 8 lanes read one whole 128-byte row
// step (a full cache line), and reads the operand layout back with
// ds_read_b128.  All loads of the main loop are these asynchronous copies, so
// the waits are exact: vmcnt counts DMA instructions only.
//   WAVES waves split K round-robin (step kt goes to wave kt % WAVES) over 16
//   weight rows per workgroup (N = 4096 gives 256 workgroups); D ring slots per
//   wave, each holding one K step of the 16 weight rows and the CB token blocks
//   (and, with block scales, that step's scale bytes); the partial sums of the
//   waves are added through LDS at the end.
//   OCC: workgroups per CU the build allows for.  Grids of at most 256
//   workgroups run one per CU (OCC = 1: the compiler may keep the
//   accumulators in AGPRs, which gave the faster loop: 7.45 against 7.74 us
//   at M = 1, N = 4096, K = 7168); larger grids share CUs two at a time.
// ---------------------------------------------------------------------------
template <int WAVES, int RB, int CB, int FA, int FB, int D, int SCL, int OCC>
__global__ __launch_bounds__(64 * WAVES, OCC) void decode_kernel(GemmParams p) {
    constexpr bool BLK = SCL == SCALE_BLOCK, CHN = SCL == SCALE_CHANNEL;
    constexpr int NB = RB + CB;                    // 16-row blocks per step: RB of weights, then CB of tokens
    constexpr int NQ = 2 * NB + (BLK ? 2 : 0);     // DMA instructions per step (8 rows x 128 B each,
                                                   // and two 256-byte scale copies)
    constexpr int SCS = BLK ? 512 : 0;             // scale bytes per slot
    constexpr int SLOT = NB * 2048 + SCS;          // bytes per ring slot
    constexpr int WRING = D * SLOT;                // bytes per wave
    static_assert(D >= 2 && NQ * (D - 1) < 64, "ring depth");
    constexpr int RED = WAVES * RB * CB * 64 * 16; // partial sums for the reduction
    constexpr int SMEM = WAVES * WRING > RED ? WAVES * WRING : RED;
    static_assert(SMEM <= 160 * 1024, "LDS");
    __shared__ __attribute__((aligned(1024))) uint8_t smem[SMEM];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // workgroup = (block of 16 RB weight rows, split of the K steps).  Split
    // K: the grid is 8 ceil(blocks / 8) x splits, workgroup (x, y) taking
    // block x and split y.  Workgroups go to the 8 XCDs in turn in the order
    // x + y 8 ceil(blocks / 8), so all splits of a block run on one XCD and
    // meet in its L2 (see the exchange below).  Those of blocks past the last
    // (live false) read nothing (no rows in their descriptors) and leave
    // before the exchange; an exit at the top made the compiler load the
    // remaining kernel arguments only after the branch, a second round of
    // scalar loads that cost every launch ~0.3 us.  Unsplit, grid y counts
    // the 64-token tiles of the small-shape class.
    const int splits = max(p.splits, 1);
    const int nb = blockIdx.x;
    const int sp = splits > 1 ? (int)blockIdx.y : 0;
    const bool live = nb < (p.N + 16 * RB - 1) / (16 * RB);
    const int n0 = nb * 16 * RB;
    const int rows_w = live ? min(p.N - n0, 16 * RB) : 0;
    // Rows past N (weights) or past M (tokens) lie outside the descriptors and
    // read zeros without touching memory.
    const v4i srdW = make_srd(p.B + (int64_t)n0 * p.ldb, rows_bytes(rows_w, p.ldb));
    // token tile: all M tokens (M <= 64), or 64-row tile blockIdx.y of them
    // (the small-shape class, never split over K)
    const int tm0 = splits > 1 ? 0 : (int)blockIdx.y * 64;
    const int rows_t = live ? min(p.M - tm0, 64) : 0;
    const v4i srdT = make_srd(p.A + (int64_t)tm0 * p.lda, rows_bytes(rows_t, p.lda));
    const int nk = (p.K + 127) / 128;
    // this split's K steps [kt0, kt1), taken by the waves round-robin
    const int kt0 = splits > 1 ? sp * p.ksteps : 0;
    const int kt1 = splits > 1 ? min(nk, kt0 + p.ksteps) : nk;
    const int nkw = kt1 - kt0;
    const int my = nkw > wave ? (nkw - wave + WAVES - 1) / WAVES : 0;   // steps kt = kt0 + wave + WAVES s
    const uint32_t ring = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t *)smem +
                          (uint32_t)wave * WRING;

    // Copy: instruction 2 b + h of a step fills rows 8 h .. 8 h + 7 of block b
    // (b = 0: weights, b = 1 + c: token block c); lane l takes row 8 h + l / 8
    // and deposits 16 bytes at position l % 8 of it, holding logical chunk
    // (l % 8) ^ key(row), key(r) = (r >> 1) & 7.  That key puts the 16 rows of
    // any one logical chunk on 16 different 16-byte bank groups for the reads.
    const uint32_t drow = (uint32_t)lane >> 3;
    const uint32_t dch0 = (((uint32_t)lane & 7u) ^ ((drow >> 1) & 7u)) * 16u;         // rows 0..7
    const uint32_t dch1 = (((uint32_t)lane & 7u) ^ (((drow + 8u) >> 1) & 7u)) * 16u;  // rows 8..15
    const uint32_t w0 = drow * (uint32_t)p.ldb + dch0, w1 = (drow + 8u) * (uint32_t)p.ldb + dch1;
    uint32_t t0[CB], t1[CB];
#pragma unroll
    for (int c = 0; c < CB; ++c) {
        t0[c] = ((uint32_t)(16 * c) + drow) * (uint32_t)p.lda + dch0;
        t1[c] = ((uint32_t)(16 * c) + drow + 8u) * (uint32_t)p.lda + dch1;
    }
    // Block scales of step kt (after the operands in the slot): the token
    // rows' scales, 4 rows per lane from scale_a[kt][0 ..], and the dword of
    // scale_b holding K block kt of the weights' 128-row block.  Token rows
    // past M may read other in-range bytes, which only reach outputs not
    // stored; reads past the arrays give zeros.
    const v4i srdSA = BLK ? make_srd(p.sfa, (uint32_t)((int64_t)nk * p.lds_sa)) : v4i{0, 0, 0, 0};
    const v4i srdSB = BLK ? make_srd(p.sfb, (uint32_t)((int64_t)((p.N + 127) / 128) * p.lds_sb)) : v4i{0, 0, 0, 0};
    const uint32_t sb_row = (uint32_t)(n0 / 128) * (uint32_t)p.lds_sb;
    auto issue = [&](int s, int slot) {
        const int kt = kt0 + wave + WAVES * s;
        const uint32_t k0 = (uint32_t)kt * 128u;
        const bool ok = s < my;
        const bool in0 = ok && (int)(k0 + dch0) < p.K, in1 = ok && (int)(k0 + dch1) < p.K;
        const uint32_t base = ring + (uint32_t)slot * SLOT;
        // The slot refilled here was read by an earlier step, and no barrier
        // separates those reads from this copy: the compiler may place that
        // step's matrix instructions, and with them the wait for its reads,
        // after this point.  So every LDS read issued so far must have
        // returned before the copy can overwrite the slot.
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
        for (int b = 0; b < RB; ++b) {
            const uint32_t wb = (uint32_t)(16 * b) * (uint32_t)p.ldb + k0;
            dma16(srdW, in0 ? w0 + wb : kOobOffset, base + 2048u * b);
            dma16(srdW, in1 ? w1 + wb : kOobOffset, base + 2048u * b + 1024u);
        }
#pragma unroll
        for (int c = 0; c < CB; ++c) {
            dma16(srdT, in0 ? t0[c] + k0 : kOobOffset, base + 2048u * (RB + c));
            dma16(srdT, in1 ? t1[c] + k0 : kOobOffset, base + 2048u * (RB + c) + 1024u);
        }
        if (BLK) {
            const uint32_t sbase = base + NB * 2048u;
            dma4(srdSA, ok && lane < 4 * CB ? (uint32_t)kt * (uint32_t)p.lds_sa + (uint32_t)tm0 + 4u * (uint32_t)lane : kOobOffset,
                 sbase);
            dma4(srdSB, ok && lane == 0 ? sb_row + ((uint32_t)kt & ~3u) : kOobOffset, sbase + 256u);
        }
    };

    // Operand reads: lane (r16, kg) = (l % 16, l / 16) takes logical chunks kg
    // and 4 + kg of row r16 of each block.
    const int r16 = lane & 15;
    const int kg = lane >> 4;
    const uint32_t rkey = ((uint32_t)r16 >> 1) & 7u;
    const uint32_t ro0 = (uint32_t)r16 * 128u + (((uint32_t)kg ^ rkey) * 16u);
    const uint32_t ro1 = (uint32_t)r16 * 128u + (((uint32_t)(4 + kg) ^ rkey) * 16u);
    const uint8_t *wbase = smem + wave * WRING;

    v4f acc[RB][CB];
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
        for (int c = 0; c < CB; ++c) acc[r][c] = (v4f){0, 0, 0, 0};
#pragma unroll
    for (int d = 0; d < D - 1; ++d) issue(d, d);
    for (int s0 = 0; s0 < my; s0 += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            // refill the slot step s - 1 used (its reads have completed: their
            // values fed the previous step's matrix instructions)
            issue(s0 + d + D - 1, (d + D - 1) % D);
            vmcnt_wait<(D - 1) * NQ>();            // step s0 + d has landed
            asm volatile("" ::: "memory");         // (and no read of it moves above the wait)
            const uint8_t *slot = wbase + d * SLOT;
            v8i wf[RB];
#pragma unroll
            for (int r = 0; r < RB; ++r)
                wf[r] = pack8(*reinterpret_cast<const v4u *>(slot + 2048 * r + ro0),
                              *reinterpret_cast<const v4u *>(slot + 2048 * r + ro1));
            const int kt = kt0 + wave + WAVES * (s0 + d);
            const int ssb = BLK ? slot[NB * 2048 + 256 + (kt & 3)] : 127;
#pragma unroll
            for (int c = 0; c < CB; ++c) {
                const uint8_t *tb = slot + 2048 * (RB + c);
                const v8i tf = pack8(*reinterpret_cast<const v4u *>(tb + ro0), *reinterpret_cast<const v4u *>(tb + ro1));
                const int ssa = BLK ? slot[NB * 2048 + c * 16 + r16] : 127;
#pragma unroll
                for (int r = 0; r < RB; ++r) {
                    if (BLK) acc[r][c] = mfma16x16x128_s<FB, FA>(wf[r], tf, acc[r][c], ssb, ssa);
                    else acc[r][c] = mfma16x16x128<FB, FA>(wf[r], tf, acc[r][c]);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    vmcnt_wait<0>();                               // drain the copies past the last step
    __syncthreads();                               // every wave's ring is idle: reuse it

    // Sum the WAVES partial accumulators (fixed order), then scale, round and
    // store: register q of a 16x16 block holds weight row 4 kg + q and token
    // column r16, so a lane writes four consecutive outputs of one token row.
    v4f *red = reinterpret_cast<v4f *>(smem);
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
        for (int c = 0; c < CB; ++c) red[((wave * RB + r) * CB + c) * 64 + lane] = acc[r][c];
    __syncthreads();
    // output block idx = (r, c): weight rows 16 r .. of this workgroup x token
    // block c; wave w takes blocks w, w + WAVES, ...
    constexpr int NBLK = RB * CB, PER = (NBLK + WAVES - 1) / WAVES;
    v4f sums[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const int idx = wave + WAVES * j;
        if (idx >= NBLK) break;
        v4f sum = red[idx * 64 + lane];
#pragma unroll
        for (int w = 1; w < WAVES; ++w) sum += red[(w * NBLK + idx) * 64 + lane];
        sums[j] = sum;
    }
    if (splits > 1) {
        if (!live) return;                         // (uniform: padding workgroup)
        // Split K: leave this split's partial sums, then count the arrival.
        // All splits of the block run on one XCD, so they meet in its L2: the
        // sums are stored plainly (the vector L1 writes through to the L2),
        // the count is an L2 atomic, and the last split reads the sums with
        // sc0 (past its L1, from the L2).  The stores have completed before
        // the count moves, so the last split sees every other split's sums.
        // Each count sits alone in a 128-byte line, so that no line is
        // updated in two XCDs' L2s, which are not coherent with each other.
        // (Sums and count written through to memory with sc0 sc1 and a
        // system-scope atomic, for splits spread over the XCDs, took 8.02
        // against 7.07 us at M = 64, N = 1024, K = 7168; device-wide fences,
        // which write back and invalidate the whole L2, were 4x slower.)  The
        // last split of the block to arrive adds all of them in split order
        // 0, 1, ..., so the result does not depend on which split finished
        // last, and resets the count for the next call.
        constexpr int kStore = 0, kLoad = 1;       // cache bits: plain store, sc0 load
        const int64_t base = (int64_t)nb * splits * NBLK * 64 * 16;
        const __amdgpu_buffer_rsrc_t part = make_rsrc(reinterpret_cast<const uint8_t *>(p.ws) + base,
                                                      (uint32_t)(splits * NBLK * 64 * 16));
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int idx = wave + WAVES * j;
            if (idx < NBLK)
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, sums[j]), part,
                                                       (uint32_t)(((sp * NBLK + idx) * 64 + lane) * 16), 0, kStore);
        }
        // (the flag takes the ring's first bytes: every wave has read its
        // share of the reduction by the first barrier below; a variable of
        // its own would take the LDS past 80 KB, one workgroup per CU)
        int *const last_split = reinterpret_cast<int *>(smem);
        vmcnt_wait<0>();                           // this thread's sums are in the L2
        __syncthreads();                           // and every thread's
        if (threadIdx.x == 0)
            *last_split = __hip_atomic_fetch_add(p.cnt + kCountStride * nb, 1, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT) == splits - 1;
        __syncthreads();
        if (!*last_split) return;
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int idx = wave + WAVES * j;
            if (idx >= NBLK) break;
            v4f sum = __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(part, (uint32_t)((idx * 64 + lane) * 16), 0, kLoad));
            for (int t = 1; t < splits; ++t)
                sum += __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(
                                                   part, (uint32_t)(((t * NBLK + idx) * 64 + lane) * 16), 0, kLoad));
            sums[j] = sum;
        }
        if (threadIdx.x == 0)
            __hip_atomic_exchange(p.cnt + kCountStride * nb, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const int idx = wave + WAVES * j;
        if (idx >= NBLK) break;
        const int r = idx / CB, c = idx % CB;
        const v4f sum = sums[j];
        const float sc = SCL != SCALE_TENSOR ? 1.0f : p.scale_a[0] * p.scale_b[0];
        const int tok = c * 16 + r16;
        if (tok < rows_t) {
            const int n = n0 + r * 16 + kg * 4;
            v2u v;
            if (CHN) {
                float s4[4], b4[4];
                channel_terms(p, n, s4, b4);
                const float sam = p.ch_sa ? p.ch_sa[tm0 + tok] : 1.0f;
                v = pack_bf16x4(sum[0] * sam * s4[0] + b4[0], sum[1] * sam * s4[1] + b4[1],
                                sum[2] * sam * s4[2] + b4[2], sum[3] * sam * s4[3] + b4[3]);
            } else {
                v = pack_bf16x4(sum[0] * sc, sum[1] * sc, sum[2] * sc, sum[3] * sc);
            }
            store_bf16x4(p.D + (int64_t)(tm0 + tok) * p.ldd, n, p.N - n, v);
        }
    }
}


// ---------------------------------------------------------------------------
// Few-token kernel with the waves on weight rows: the dense form with M <= 64
// where the weight rows are few enough that K is split over workgroups
// anyway.  Wave w owns weight rows 64 b + 16 w .. +16 of the workgroup's
// block b, and the 4 waves share one LDS ring of token rows: each K step's
// tokens are copied once for 64 weight rows, where the waves-on-K kernel
// above copies them once for 16.  Every 1 KB direct-to-LDS copy costs the
// texture addresser 16 cycles, so at M = 64 (4 token blocks) the token
// copies are four fifths of that kernel's copy instructions; with the token
// and weight copies aimed out of range (no memory traffic) it still took
// 6.45 us at M = 64, N = 4096, K = 7168 against 4.0 at M = 1.
//   K: grid y splits the K steps (`ksteps` each) as in the kernel above, the
//   grid x padded to a multiple of 8 so that all splits of a block run on
//   one XCD and meet in its L2; every wave runs all of its split's steps.
//   Ring: TS = LT + 1 token slots shared by the waves and LT + 2 weight
//   slots per wave.  The copies of step s + LT (tokens, L2 hits) and of step
//   s + LT + 1 (this wave's weights, from HBM) are issued after step s's
//   barrier, tokens first, so the weights run one step further ahead and the
//   wait before a step leaves the newest weight copies in flight (copies
//   complete in issue order).
// ---------------------------------------------------------------------------
template <int CB, int SCL, int LT>
struct RowsDecodeLayout {
    static constexpr bool BLK = SCL == SCALE_BLOCK;
    static constexpr int TR = CB <= 2 ? 32 : 16 * CB;   // token rows per step (>= 32: one copy per wave)
    static constexpr int TDMA = TR / 32;                // token copies per wave per step (8 rows each)
    static constexpr int TS = LT + 1;                   // token slots
    static constexpr int DW = LT + 2;                   // weight slots per wave
    static constexpr int TSLOT = TR * 128;
    static constexpr int WSLOT = 16 * 128;
    static constexpr int SCS = BLK ? 256 : 0;           // token-scale bytes per token slot
    static constexpr int WSC = BLK ? 256 : 0;           // weight-scale bytes per weight slot
    static constexpr int T_OFF = 4 * DW * WSLOT;        // [weight rings | token ring | token scales |
    static constexpr int TSC_OFF = T_OFF + TS * TSLOT;  //  weight scales | arrival flag]
    static constexpr int WSC_OFF = TSC_OFF + TS * SCS;
    static constexpr int FLAG_OFF = WSC_OFF + 4 * DW * WSC;
    static constexpr int SMEM = FLAG_OFF + 16;
};

template <int CB, int FA, int FB, int SCL, int LT, int OCC>
__global__ __launch_bounds__(256, OCC) void decode_rows_kernel(GemmParams p) {
    using L = RowsDecodeLayout<CB, SCL, LT>;
    constexpr bool BLK = L::BLK, CHN = SCL == SCALE_CHANNEL;
    constexpr int TDMA = L::TDMA, TS = L::TS, DW = L::DW;
    constexpr int WLOADS = 2 + (BLK ? 1 : 0);      // this wave's weight copies (and block scale) per step
    constexpr int SDMA = BLK ? 1 : 0;              // wave 0: the token rows' scales per step
    constexpr int WAIT = WLOADS + (LT - 1) * (TDMA + WLOADS);
    constexpr int WAIT0 = WLOADS + (LT - 1) * (TDMA + SDMA + WLOADS);
    static_assert(LT >= 1 && WAIT0 < 64, "copies in flight");
    static_assert(L::SMEM <= 160 * 1024, "LDS");
    __shared__ __attribute__((aligned(1024))) uint8_t smem[L::SMEM];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // workgroup (x, y) = (block of 64 weight rows, split of the K steps);
    // blocks past the last (padding of the grid x) read nothing and leave
    // before the exchange
    const int splits = max(p.splits, 1);
    const int nb = blockIdx.x;
    const int sp = splits > 1 ? (int)blockIdx.y : 0;
    const bool live = nb < (p.N + 63) / 64;
    const int nw = nb * 64 + wave * 16;            // this wave's first weight row
    const int rows_w = live ? max(0, min(p.N - nw, 16)) : 0;
    const int rows_t = live ? p.M : 0;
    // Rows past N (weights) or past M (tokens) lie outside the descriptors and
    // read zeros without touching memory.
    const v4i srdW = make_srd(p.B + (int64_t)min(nw, p.N) * p.ldb, rows_bytes(rows_w, p.ldb));
    const v4i srdT = make_srd(p.A, rows_bytes(rows_t, p.lda));
    const int nk = (p.K + 127) / 128;
    const int kt0 = splits > 1 ? sp * p.ksteps : 0;
    const int nks = splits > 1 ? max(0, min(nk, kt0 + p.ksteps) - kt0) : nk;
    // Block scales: the token rows' scales of K block kt at sfa[kt lds_sa ..],
    // and the dword of scale_b holding K block kt of the 128-row scale block
    // that this workgroup's 64 rows lie in.
    const v4i srdSA = BLK ? make_srd(p.sfa, (uint32_t)((int64_t)nk * p.lds_sa)) : v4i{0, 0, 0, 0};
    const v4i srdSB = BLK ? make_srd(p.sfb, (uint32_t)((int64_t)((p.N + 127) / 128) * p.lds_sb)) : v4i{0, 0, 0, 0};
    const uint32_t sb_row = BLK ? (uint32_t)(min(nb * 64, p.N) / 128) * (uint32_t)p.lds_sb : 0u;
    const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t *)smem;
    const uint32_t wring = lds0 + (uint32_t)(wave * DW * L::WSLOT);

    // Weight copies: instruction h fills rows 8 h .. 8 h + 7 of the wave's
    // slot; lane l takes row 8 h + l / 8 and deposits 16 bytes at position
    // l % 8 of it, holding logical chunk (l % 8) ^ ((row >> 1) & 7), which puts
    // the 16 rows of one logical chunk on 16 different bank groups for the
    // fragment reads.
    const uint32_t wrow = (uint32_t)lane >> 3;
    const uint32_t wch0 = (((uint32_t)lane & 7u) ^ ((wrow >> 1) & 7u)) * 16u;
    const uint32_t wch1 = (((uint32_t)lane & 7u) ^ (((wrow + 8u) >> 1) & 7u)) * 16u;
    const uint32_t wo0 = wrow * (uint32_t)p.ldb + wch0, wo1 = (wrow + 8u) * (uint32_t)p.ldb + wch1;
    const int r16 = lane & 15;
    const int kg = lane >> 4;
    const uint32_t wkey = ((uint32_t)r16 >> 1) & 7u;
    const uint32_t wf0 = (uint32_t)r16 * 128u + (((uint32_t)kg ^ wkey) * 16u);
    const uint32_t wf1 = (uint32_t)r16 * 128u + (((uint32_t)(4 + kg) ^ wkey) * 16u);
    // Token copies: instruction i of wave w fills token rows (w TDMA + i) 8 ..
    // +8 of the slot, lane l row l / 8, position l % 8 holding logical chunk
    // (l % 8) ^ ((row >> 1) & 7), the weights' key: the fragment reads of any
    // 16 rows are then free of bank conflicts.  (The key (r & 7) ^ ((r >> 3) &
    // 1) of swz() left 44% of the LDS-active cycles in conflicts here.)
    uint32_t t_off[TDMA], t_kc[TDMA];
#pragma unroll
    for (int i = 0; i < TDMA; ++i) {
        const uint32_t row = (uint32_t)((wave * TDMA + i) * 8 + (lane >> 3));
        const uint32_t c = ((uint32_t)(lane & 7) ^ ((row >> 1) & 7u)) & 7u;
        t_kc[i] = c * 16u;
        t_off[i] = row * (uint32_t)p.lda + c * 16u;
    }
    uint32_t t_frag[CB][2];
#pragma unroll
    for (int c = 0; c < CB; ++c) {
        const uint32_t row = (uint32_t)(c * 16 + r16);
        const uint32_t key = (row >> 1) & 7u;
        t_frag[c][0] = row * 128u + ((((uint32_t)kg) ^ key) & 7u) * 16u;
        t_frag[c][1] = row * 128u + ((((uint32_t)kg + 4u) ^ key) & 7u) * 16u;
    }

    // The copies of local step s (K block kt0 + s); past the split's last step
    // every offset is out of range: zeros, no traffic, never consumed.
    auto load_w = [&](int s) {
        const int kt = kt0 + s;
        const uint32_t k0 = (uint32_t)kt * 128u;
        const bool ok = s < nks;
        const bool in0 = ok && (int)(k0 + wch0) < p.K, in1 = ok && (int)(k0 + wch1) < p.K;
        const uint32_t dst = wring + (uint32_t)((s % DW) * L::WSLOT);
        dma16(srdW, in0 ? wo0 + k0 : kOobOffset, dst);
        dma16(srdW, in1 ? wo1 + k0 : kOobOffset, dst + 1024u);
        if (BLK)
            dma4(srdSB, ok && lane == 0 ? sb_row + ((uint32_t)kt & ~3u) : kOobOffset,
                 lds0 + (uint32_t)(L::WSC_OFF + (wave * DW + s % DW) * L::WSC));
    };
    auto load_t = [&](int s) {
        const int kt = kt0 + s;
        const uint32_t k0 = (uint32_t)kt * 128u;
        const bool ok = s < nks;
        const uint32_t dst = lds0 + (uint32_t)(L::T_OFF + (s % TS) * L::TSLOT);
#pragma unroll
        for (int i = 0; i < TDMA; ++i) {
            const bool in = ok && (int)(k0 + t_kc[i]) < p.K;
            dma16(srdT, in ? t_off[i] + k0 : kOobOffset, dst + (uint32_t)(wave * TDMA + i) * 1024u);
        }
        if (BLK && wave == 0)
            dma4(srdSA, ok && 4 * lane < 16 * CB ? (uint32_t)kt * (uint32_t)p.lds_sa + 4u * (uint32_t)lane : kOobOffset,
                 lds0 + (uint32_t)(L::TSC_OFF + (s % TS) * L::SCS));
    };

    v4f acc[CB];
#pragma unroll
    for (int c = 0; c < CB; ++c) acc[c] = (v4f){0, 0, 0, 0};
    // issue order: W0 | T0 W1 | ... | T(LT-1) W(LT), then per step s after its
    // barrier T(s+LT) W(s+LT+1)
    load_w(0);
#pragma unroll
    for (int j = 0; j < LT; ++j) {
        load_t(j);
        load_w(j + 1);
    }
    __builtin_amdgcn_sched_barrier(0);
    for (int s = 0; s < nks; ++s) {
        // every copy of step s has landed (this wave's), then every wave's; the
        // slots of step s - 1 are no longer read
        if (BLK && wave == 0) vmcnt_wait<WAIT0>();
        else vmcnt_wait<WAIT>();
        __syncthreads();
        load_t(s + LT);
        load_w(s + LT + 1);
        __builtin_amdgcn_sched_barrier(0);
        const uint8_t *ts = smem + L::T_OFF + (s % TS) * L::TSLOT;
        const uint8_t *ws = smem + (wave * DW + s % DW) * L::WSLOT;
        const v8i wf = pack8(*reinterpret_cast<const v4u *>(ws + wf0), *reinterpret_cast<const v4u *>(ws + wf1));
        const int ssb = BLK ? (int)smem[L::WSC_OFF + (wave * DW + s % DW) * L::WSC + ((kt0 + s) & 3)] : 127;
#pragma unroll
        for (int c = 0; c < CB; ++c) {
            const v8i tf = pack8(*reinterpret_cast<const v4u *>(ts + t_frag[c][0]),
                                 *reinterpret_cast<const v4u *>(ts + t_frag[c][1]));
            const int ssa = BLK ? (int)smem[L::TSC_OFF + (s % TS) * L::SCS + c * 16 + r16] : 127;
            if (BLK) acc[c] = mfma16x16x128_s<FB, FA>(wf, tf, acc[c], ssb, ssa);
            else acc[c] = mfma16x16x128<FB, FA>(wf, tf, acc[c]);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    vmcnt_wait<0>();                               // drain the copies past the last step

    if (splits > 1) {
        if (!live) return;                         // (uniform: padding workgroup)
        // Split K, as in the kernel above: this split's sums stored plainly
        // (the vector L1 writes through to the XCD's L2), the arrival counted
        // with an L2 atomic on the block's own 128-byte line, and the last
        // split to arrive adds every split's sums, read with sc0 from the L2,
        // in split order, then resets the count.
        constexpr int kStore = 0, kLoad = 1;
        constexpr int PART = 4 * CB * 1024;        // one split's sums: 4 waves x CB blocks x 64 lanes x 16 B
        const __amdgpu_buffer_rsrc_t part =
            make_rsrc(reinterpret_cast<const uint8_t *>(p.ws) + (int64_t)nb * splits * PART, (uint32_t)(splits * PART));
#pragma unroll
        for (int c = 0; c < CB; ++c)
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, acc[c]), part,
                                                   (uint32_t)(sp * PART + (wave * CB + c) * 1024 + lane * 16), 0, kStore);
        int *const last_split = reinterpret_cast<int *>(smem + L::FLAG_OFF);
        vmcnt_wait<0>();                           // this thread's sums are in the L2
        __syncthreads();                           // and every thread's
        if (threadIdx.x == 0)
            *last_split = __hip_atomic_fetch_add(p.cnt + kCountStride * nb, 1, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT) == splits - 1;
        __syncthreads();
        if (!*last_split) return;
#pragma unroll
        for (int c = 0; c < CB; ++c) {
            const uint32_t off = (uint32_t)((wave * CB + c) * 1024 + lane * 16);
            v4f sum = __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(part, off, 0, kLoad));
            for (int t = 1; t < splits; ++t)
                sum += __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(part, (uint32_t)(t * PART) + off, 0, kLoad));
            acc[c] = sum;
        }
        if (threadIdx.x == 0)
            __hip_atomic_exchange(p.cnt + kCountStride * nb, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    // Scale, round, store: register q of block c holds weight row nw + 4 kg + q
    // and token c 16 + r16, so a lane writes four consecutive outputs of one
    // token row.
    const float sc = SCL != SCALE_TENSOR ? 1.0f : p.scale_a[0] * p.scale_b[0];
    const int n = nw + kg * 4;
#pragma unroll
    for (int c = 0; c < CB; ++c) {
        const int tok = c * 16 + r16;
        if (tok < rows_t) {
            const v4f sum = acc[c];
            v2u v;
            if (CHN) {
                float s4[4], b4[4];
                channel_terms(p, n, s4, b4);
                const float sam = p.ch_sa ? p.ch_sa[tok] : 1.0f;
                v = pack_bf16x4(sum[0] * sam * s4[0] + b4[0], sum[1] * sam * s4[1] + b4[1],
                                sum[2] * sam * s4[2] + b4[2], sum[3] * sam * s4[3] + b4[3]);
            } else {
                v = pack_bf16x4(sum[0] * sc, sum[1] * sc, sum[2] * sc, sum[3] * sc);
            }
            store_bf16x4(p.D + (int64_t)tok * p.ldd, n, p.N - n, v);
        }
    }
}

}  // namespace fp8g
