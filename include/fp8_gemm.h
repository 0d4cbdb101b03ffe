/*
 * fp8_gemm.h -- C ABI of the MI355X (gfx950) FP8 GEMM library.
 *
 * Computes D = bf16( scale_a * scale_b * A . B^T ) with FP8 operands (E4M3 or
 * E5M2, chosen per operand), FP32 accumulation on the CDNA4 matrix cores, and a
 * fused epilogue that applies the per-tensor scales and rounds to BF16.
 *
 * Sources on the pages:
 *   - "DeepGEMM: FP8 matrix-multiply kernels on Hopper Tensor Cores":
 *       section 1.3 and 3.1 (FP8 E4M3/E5M2 inputs, FP32 accumulator, the scale
 *       multiplied back once at the output), section 2.1 (what one output
 *       element is), section 5.2 (per-tensor scales), section 6.4 (alignment
 *       matters; no unordered FP32 atomics, so results are deterministic).
 *   - "One transpose, half the compute: the DeepSeek SwapAB story":
 *       section 2 (MoE decode: each expert sees only tens of tokens),
 *       section 3.1 (the masked grouped FP8 GEMM, "nt" layout: both operands
 *       K-contiguous), section 3.2-3.3 (operands swapped so weights take the
 *       rigid side and the tokens the flexible side; work shrinks to the
 *       valid rows), section 3.5 (the swap is chosen on the host from the
 *       per-expert token count).
 *
 * Conventions for every entry point:
 *   - All pointers except `stream` are DEVICE pointers (memory the caller
 *     allocated, e.g. through PyTorch).  The caller owns every buffer it
 *     passes; the library keeps no pointer to them after returning and never
 *     synchronises the stream.
 *   - Workspace: the dense forms with M <= 64 split K over workgroups when
 *     the weight rows alone would leave the chip part-empty or unevenly
 *     loaded (fewer than 256 blocks of 16 rows, or 64-row blocks; at most
 *     256 blocks and 512 workgroups).  The splits' FP32 partial sums meet in a
 *     workspace of 8 MiB + 32 KiB per device, which the library allocates
 *     with hipMalloc on the first such call on that device (and keeps until
 *     the process ends); if that first call happens while `stream` is being
 *     captured into a graph, it runs unsplit instead (nothing allocated; the
 *     same bound holds, though the FP32 sums are added in another order).
 *     The partial sums are added in a fixed order, so repeated calls give
 *     bit-identical results whichever split finishes last.  Calls that split K and overlap
 *     on one device (different streams or threads without ordering) share
 *     the workspace and race: order them.  No other path uses device memory
 *     beyond the caller's buffers.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream).
 *     Results are valid once that stream's work has completed.
 *   - FP8 operands are byte arrays of codes; dtypes are FP8G_E4M3 (OCP E4M3FN:
 *     max 448, S.1111.111 = NaN, no infinities) or FP8G_E5M2 (OCP E5M2).
 *   - D is BF16 (uint16 bit patterns), rounded to nearest even.  D must not
 *     alias A, B, the scales or the index vectors.
 *   - Arguments are validated before anything is enqueued.  A nonzero return
 *     (an fp8g_status) from validation means nothing was enqueued;
 *     fp8_gemm_strerror() gives the reason, including a per-thread detail
 *     string for the last failure.
 *   - Zero-sized problems (M, N, G, cap or M_total = 0) return FP8G_OK and
 *     enqueue nothing.  K = 0 writes zeros (the empty sum); A and B may then be
 *     NULL, as nothing is read from them.
 *   - Limits: K % 16 == 0; A, B, D pointers 16-byte aligned; row strides in
 *     bytes (A, B) multiples of 16 and at most 2^23 - 16; ldd a multiple of 8
 *     elements (the grouped forms use ldd = N, so N % 8 == 0 there); M, N, K,
 *     G, cap, M_total below 2^31.
 *   - Values that live on the device (masked_m, grp_idx) cannot be checked
 *     without a synchronisation: masked_m[g] is clamped to [0, cap], and any
 *     grp_idx entry outside [0, G) marks a padding row.
 *   - Results are deterministic: no floating-point atomics; the same call on
 *     the same inputs gives bit-identical D.
 */
#ifndef FP8_GEMM_H
#define FP8_GEMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FP8G_ABI_VERSION 4

typedef enum { FP8G_E4M3 = 0, FP8G_E5M2 = 1 } fp8g_dtype;

typedef enum {
    FP8G_OK = 0,
    FP8G_ERR_NULL = -1,         /* a required pointer is NULL */
    FP8G_ERR_SHAPE = -2,        /* negative or too large size, K % 16 != 0 */
    FP8G_ERR_ALIGN = -3,        /* pointer or stride not 16-byte aligned */
    FP8G_ERR_DTYPE = -4,        /* dtype is neither FP8G_E4M3 nor FP8G_E5M2 */
    FP8G_ERR_STRIDE = -5,       /* lda/ldb < K, ldd < N, or stride too large */
    FP8G_ERR_LAUNCH = -6,       /* the HIP launch reported an error */
    FP8G_ERR_UNSUPPORTED = -7,  /* no device of the supported architecture */
    FP8G_ERR_ARG = -8           /* any other invalid argument (e.g. expected_m > cap) */
} fp8g_status;

/*
 * Dense GEMM, "nt" layout.
 *   A: [M x K] FP8 codes, row stride lda bytes (K contiguous).
 *   B: [N x K] FP8 codes, row stride ldb bytes (K contiguous).
 *   scale_a, scale_b: one FP32 each (device).
 *   D: [M x N] BF16, row stride ldd elements.
 *   D[i][j] = bf16_rne( (scale_a * scale_b) * sum_k A[i][k] * B[j][k] ).
 * M <= 64 takes the swapped (weights-on-rows, tokens-on-columns) decode
 * kernel, with K split over workgroups when the weight rows are few (see
 * Workspace above); larger M takes the LDS-tiled kernel.  The choice never
 * changes which elements are written.
 */
int fp8_gemm_nt(const void *A, int64_t lda, int a_dtype,
                const void *B, int64_t ldb, int b_dtype,
                const float *scale_a, const float *scale_b,
                void *D, int64_t ldd,
                int M, int N, int K, void *stream);

/*
 * fp8_gemm_nt for callers that cannot allocate device memory (code under
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same arguments, kernels and results, but the split-K few-token path keeps
 * its partial sums in a fixed scratch array inside the library's code object
 * (8 MiB of FP32 sums and 256 arrival counts of 128 bytes each per device,
 * 8 MiB + 32 KiB, held from the
 * library's load until the process ends) instead of a workspace allocated on
 * first use.  It calls no allocation routine.  Every shape fits the array
 * (the split-K path splits at most 256 blocks of weight rows over at most
 * 512 workgroups of at most 16 KiB of sums); a larger need would be refused
 * with FP8G_ERR_ARG.  All calls on a
 * device share its array, which keeps the last call's contents (the counts
 * return to zero after every call): calls that overlap on one device race.
 */
int fp8_gemm_nt_noalloc(const void *A, int64_t lda, int a_dtype,
                        const void *B, int64_t ldb, int b_dtype,
                        const float *scale_a, const float *scale_b,
                        void *D, int64_t ldd,
                        int M, int N, int K, void *stream);

/*
 * Block-scaled dense GEMM, "nt" layout, with power-of-two block scales: one
 * per row of A and 128-element block of K, one per 128 rows of B and
 * 128-element block of K ("DeepGEMM: FP8 matrix-multiply kernels on Hopper
 * Tensor Cores", section 5.2: scales per group of 128 elements; "One
 * transpose, half the compute: the DeepSeek SwapAB story", section 5: UE8M0
 * packed scales).
 *   A, B, D, lda, ldb, ldd, M, N, K: as for fp8_gemm_nt.
 *   scale_a: E8M0 codes (uint8, device), [ceil(K/128)][lds_a]: the scale of row
 *     m of A over K block kb is 2^(scale_a[kb * lds_a + m] - 127).
 *     lds_a >= M, lds_a % 4 == 0 (rows M .. lds_a-1 are never used).
 *   scale_b: E8M0 codes (uint8, device), [ceil(N/128)][lds_b]: the scale of
 *     rows 128 nb .. 128 nb + 127 of B over K block kb is
 *     2^(scale_b[nb * lds_b + kb] - 127).  lds_b >= ceil(K/128), lds_b % 4 == 0.
 *   Code 255 is NaN and makes every output element whose sum it scales NaN.
 *   Both scale pointers 4-byte aligned; each array below 2^31 bytes.
 *   D[i][j] = bf16_rne( sum_kb 2^(ea(i,kb) - 127) * 2^(eb(j/128,kb) - 127)
 *                        * sum_{k in block kb} A[i][k] * B[j][k] ).
 * The scales are exact powers of two, applied to the products inside the
 * matrix-core instruction, so they cost no arithmetic.  M <= 64 takes the
 * swapped decode kernel, larger M the LDS-tiled kernel.
 */
int fp8_gemm_nt_blockscaled(const void *A, int64_t lda, int a_dtype,
                            const void *B, int64_t ldb, int b_dtype,
                            const uint8_t *scale_a, int64_t lds_a,
                            const uint8_t *scale_b, int64_t lds_b,
                            void *D, int64_t ldd,
                            int M, int N, int K, void *stream);

/*
 * Dense GEMM with per-row and per-channel scales and a per-channel bias
 * ("DeepGEMM: FP8 matrix-multiply kernels on Hopper Tensor Cores", section 5.2:
 * a scale per channel instead of one per tensor; the bias is the additive term
 * of a fused epilogue).
 *   A, B, D, lda, ldb, ldd, M, N, K: as for fp8_gemm_nt.
 *   scale_a: [M] floats (device, 4-byte aligned), one per row of A (token), or NULL = 1.
 *   scale_b: [N] floats (device, 16-byte aligned), one per output channel, or NULL = 1.
 *   bias:    [N] floats (device, 16-byte aligned), or NULL = 0.
 *   D[i][j] = bf16_rne( scale_a[i] * scale_b[j] * sum_k A[i][k] * B[j][k] + bias[j] ),
 *   the scale and bias applied in FP32 to the FP32 accumulator.
 * Same kernels and shape classes as fp8_gemm_nt.
 */
int fp8_gemm_nt_channelwise(const void *A, int64_t lda, int a_dtype,
                            const void *B, int64_t ldb, int b_dtype,
                            const float *scale_a, const float *scale_b, const float *bias,
                            void *D, int64_t ldd,
                            int M, int N, int K, void *stream);

/*
 * BF16 comparison GEMM ("DeepGEMM: FP8 matrix-multiply kernels on Hopper
 * Tensor Cores", section 1.3: the backend keeps a BF16 path for precision
 * experiments beside the default FP8 path).
 *   A: [M][lda] BF16 (device), K-contiguous rows; B: [N][ldb] BF16 (device).
 *   D: [M][ldd] BF16 (device).
 *   D[i][j] = bf16_rne( sum_k A[i][k] * B[j][k] ): no scales; the products are
 *     exact and the matrix cores sum them in FP32.
 *   Strides in elements: lda, ldb >= K and multiples of 8 (16 bytes), at most
 *     (2^23 - 16) / 2; ldd >= N, a multiple of 8.  K % 8 == 0.  A, B, D
 *     16-byte aligned.  K = 0 writes zeros.
 * Runs on the 8-wave LDS-tiled kernel of the grouped forms, for every M, with
 * the tile chosen as for the FP8 dense form: it stages the same bytes, and
 * each 32-byte fragment feeds two BF16 instructions instead of one FP8
 * instruction.
 */
int bf16_gemm_nt(const void *A, int64_t lda, const void *B, int64_t ldb,
                 void *D, int64_t ldd, int M, int N, int K, void *stream);

/*
 * Masked grouped GEMM (MoE decode).
 *   A: [G][cap][K] FP8 codes, contiguous.  B: [G][N][K] FP8 codes, contiguous.
 *   masked_m: [G] int32 (device); group g has m_g = clamp(masked_m[g], 0, cap)
 *     valid rows.
 *   scale_a: 1 float; scale_b: [G] floats (device), one per expert.
 *   D: [G][cap][N] BF16, contiguous.
 *   For i < m_g: D[g][i][j] = bf16_rne( (scale_a * scale_b[g]) * sum_k A[g][i][k] * B[g][j][k] ).
 *   Rows i >= m_g of A are never read and rows i >= m_g of D are never written.
 *   A group with m_g = 0 reads nothing.
 *   expected_m: host hint of the typical m_g, 0 <= expected_m <= cap (0 = use
 *     cap).  It only picks the kernel variant and never changes results: up
 *     to 192 the swapped streaming kernel, which reads each group's weights
 *     once for up to 16 (1..16), 32, 64, 128 or 192 (129..192) tokens and
 *     loops over token blocks when a group has more; above 192 the tiled
 *     kernel with 128-row tiles.
 */
int fp8_grouped_gemm_masked(const void *A, int a_dtype, const void *B, int b_dtype,
                            const float *scale_a, const float *scale_b,
                            const int32_t *masked_m, void *D,
                            int G, int cap, int N, int K, int expected_m, void *stream);

/*
 * Block-scaled masked grouped GEMM (MoE decode with the block-scaled format of
 * fp8_gemm_nt_blockscaled, per expert).
 *   A, B, masked_m, D, G, cap, N, K, expected_m: as for fp8_grouped_gemm_masked.
 *   scale_a: E8M0 codes (uint8, device), [G][ceil(K/128)][lds_a]: the scale of
 *     row i of group g over K block kb is 2^(scale_a[(g * ceil(K/128) + kb) * lds_a + i] - 127).
 *     lds_a >= cap, lds_a % 4 == 0.
 *   scale_b: E8M0 codes (uint8, device), [G][ceil(N/128)][lds_b]: rows
 *     128 nb .. 128 nb + 127 of B[g] over K block kb at
 *     scale_b[(g * ceil(N/128) + nb) * lds_b + kb].  lds_b >= ceil(K/128), lds_b % 4 == 0.
 *   Code 255 is NaN.  Scale arrays 4-byte aligned; each group's below 2^31 bytes.
 *   For i < m_g: D[g][i][j] = bf16_rne( sum_kb 2^(ea - 127) 2^(eb - 127) sum_{k in kb} A[g][i][k] B[g][j][k] ).
 *   Rows i >= m_g of A are never read and rows i >= m_g of D never written;
 *   their scale bytes may be read and never reach a written output.
 */
int fp8_grouped_gemm_masked_blockscaled(const void *A, int a_dtype, const void *B, int b_dtype,
                                        const uint8_t *scale_a, int64_t lds_a,
                                        const uint8_t *scale_b, int64_t lds_b,
                                        const int32_t *masked_m, void *D,
                                        int G, int cap, int N, int K, int expected_m, void *stream);

/*
 * Contiguous grouped GEMM (MoE prefill).
 *   A: [M_total][K] FP8 codes, contiguous; the rows of each expert are
 *     contiguous and each expert's run starts on a multiple of 128 rows
 *     (padding rows fill each run up to the next multiple of 128).
 *   B: [G][N][K] FP8 codes, contiguous.  scale_a: 1 float; scale_b: [G] floats.
 *   grp_idx: [M_total] int32 (device).  Row r with 0 <= grp_idx[r] < G uses
 *     expert grp_idx[r]; any other value marks a padding row, which is not
 *     written.  Every aligned block of 128 rows must hold rows of at most one
 *     expert (plus padding); rows of a second expert inside a block are left
 *     unwritten.
 *   D: [M_total][N] BF16, contiguous.
 * Work is split into tiles of 256 rows: a tile computes the rows of the
 * expert of its first valid row; a second set of workgroups, one per tile,
 * computes a tile's second 128-row block when it belongs to another expert.
 */
int fp8_grouped_gemm_contig(const void *A, int a_dtype, const void *B, int b_dtype,
                            const float *scale_a, const float *scale_b,
                            const int32_t *grp_idx, void *D,
                            int M_total, int G, int N, int K, void *stream);

/*
 * Block-scaled contiguous grouped GEMM (MoE prefill with the block-scaled
 * format of fp8_gemm_nt_blockscaled).
 *   A, B, grp_idx, D, M_total, G, N, K: as for fp8_grouped_gemm_contig.
 *   scale_a: E8M0 codes (uint8, device), [ceil(K/128)][lds_a]: the scale of row
 *     r of A over K block kb at scale_a[kb * lds_a + r].  lds_a >= M_total,
 *     lds_a % 4 == 0.
 *   scale_b: E8M0 codes (uint8, device), [G][ceil(N/128)][lds_b]: rows
 *     128 nb .. 128 nb + 127 of expert e over K block kb at
 *     scale_b[(e * ceil(N/128) + nb) * lds_b + kb].  lds_b >= ceil(K/128), lds_b % 4 == 0.
 *   Code 255 is NaN.  Scale arrays 4-byte aligned and below 2^31 bytes (per expert for scale_b).
 *   Row r with a valid expert e = grp_idx[r]:
 *     D[r][j] = bf16_rne( sum_kb 2^(ea(r,kb) - 127) 2^(eb(e,j/128,kb) - 127) sum_{k in kb} A[r][k] B[e][j][k] ).
 *   Padding rows are not written; their scale bytes may be read.
 * Work is split into tiles aligned to each expert's run of 128-row blocks:
 * 256 rows, and 128 rows at the end of a run with an odd number of blocks, so
 * no block is computed twice.  The runs are found on the device (the counts
 * never pass through the host); a block's expert is that of its first row
 * naming a valid expert.
 */
int fp8_grouped_gemm_contig_blockscaled(const void *A, int a_dtype, const void *B, int b_dtype,
                                        const uint8_t *scale_a, int64_t lds_a,
                                        const uint8_t *scale_b, int64_t lds_b,
                                        const int32_t *grp_idx, void *D,
                                        int M_total, int G, int N, int K, void *stream);

/*
 * Kernel choice for a problem, without launching anything (host only).
 *   op: 0 = dense (m = M), 1 = masked grouped (m = cap, hint = expected_m,
 *   groups = G), 2 = contiguous grouped (m = M_total, groups = G),
 *   3 = block-scaled dense (m = M), 4 = BF16 dense (m = M, k in BF16
 *   elements), 5 = block-scaled contiguous grouped (m = M_total, groups = G).
 * Fills the variant id, the tile sizes along M and N, and the number of
 * workgroups of the launch.  Returns an fp8g_status (validation as above,
 * pointers excepted).
 */
typedef struct {
    int variant;        /* 1 = tiled 256x256, 2 = tiled 128x256 (m x n; FP8
                           dense forms on 4 waves and 16x16x128, grouped and
                           BF16 forms on 8 waves and 32x32x64),
                           3 = swapped streaming (masked grouped forms,
                           16 * token_blocks tokens per pass),
                           4 = swapped decode (dense forms, m <= 64): 16
                           or 32 weight rows per workgroup with K split over
                           its 4 waves, or 64 with each wave on 16 of them;
                           K also split over k_splits workgroups, 5 = tiled 256x192 and
                           6 = tiled 256x224 (both FP8 dense, per-tensor or
                           per-channel scales), 0 = nothing to launch */
    int tile_m;         /* rows of D per workgroup tile (tokens) */
    int tile_n;         /* columns of D per workgroup tile (weight rows: 256
                           or 512 for variant 3, 16, 32 or 64 for variant 4) */
    int token_blocks;   /* swapped kernels: 16-token column blocks per pass
                           (1, 2, 4; the masked form also 8 and 12) */
    int64_t workgroups; /* grid size */
    int k_splits;       /* variant 4: workgroups sharing one block of weight
                           rows, each over a part of K (1 = no split) */
} fp8g_plan;

int fp8_gemm_plan(int op, int m, int n, int k, int groups, int expected_m, fp8g_plan *out);

/* Human-readable text for a status, followed by the calling thread's detail
 * for its last failed call (the returned pointer stays valid until that
 * thread's next call into the library). */
const char *fp8_gemm_strerror(int status);

/* FP8G_ABI_VERSION of the built library. */
int fp8_gemm_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FP8_GEMM_H */
