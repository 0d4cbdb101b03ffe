/*
 * Plain CPU oracle for FP8 GEMM  D = bf16( sa * sb * A . B^T ).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link or
 * call this file: only the test suite, the smoke check and the CPU-baseline leg
 * of the benchmark use it.  It shares no code, header, table or helper with the
 * HIP library.
 *
 * What it computes, and where that is stated:
 *   - "DeepGEMM: FP8 matrix-multiply kernels on Hopper Tensor Cores", section 2.1:
 *     the naive triple loop, one output element C[i][j] as the inner product of
 *     row i of A with column j of the (here transposed, K-major) B.
 *   - same page, section 3.1: inputs are FP8 in E4M3 (4 exponent, 3 mantissa
 *     bits) or E5M2 (5 exponent, 2 mantissa bits); accumulation is in a wider
 *     format; the per-tensor scale is applied once at the output, not per element.
 *   - same page, section 5.2: per-tensor scales.
 *   - "One transpose, half the compute: the DeepSeek SwapAB story", sections 2
 *     and 3.1-3.3: the masked grouped GEMM over experts, each expert with its own
 *     count of valid token rows; only valid rows are computed.
 *
 * Readings where the pages are silent (each is listed with its reason in the
 * design notes):
 *   - FP8 flavour: OCP E4M3FN (no infinities, S.1111.111 is NaN, max 448) and
 *     OCP E5M2 (IEEE-like, inf and NaN at exponent 31, max 57344); subnormals
 *     are decoded, not flushed.
 *   - Accumulation in FP64, sequential in k.  For E4M3 x E4M3 this is exact
 *     (every product is an integer multiple of 2^-18 below 2^36 in magnitude).
 *     An independent integer (__int128) accumulation reports, per element,
 *     whether the FP64 sum equals the exact sum.
 *   - Scale: r = acc * ((double)sa * (double)sb); the scale product is exact
 *     in FP64, so r carries one rounding beyond acc.
 *   - Output rounding: BF16 round-to-nearest-even, directly from the double
 *     (one rounding); overflow goes to +-inf; NaN becomes 0x7FC0.
 *   - Masked grouped: rows i < clamp(masked_m[g], 0, cap) are computed, other
 *     rows of D are not touched.
 *   - Contiguous grouped: row r with 0 <= grp_idx[r] < G uses expert grp_idx[r]
 *     and scale_b[grp_idx[r]]; other rows are padding and are not touched.
 *   - Block-scaled dense (DeepGEMM on Hopper, section 5.2: scales per group of
 *     128 elements; "One transpose, half the compute", section 5: UE8M0 packed
 *     scales): A has one scale per (row, block of 128 along K), B one per
 *     (block of 128 rows, block of 128 along K).  Each scale is an unsigned
 *     E8M0 code e, value 2^(e - 127); e = 255 is NaN.  A K block's partial
 *     sum is multiplied by the two scales of its block and added to the
 *     accumulator: acc = sum_kb sa(m,kb) * sb(n/128,kb) * sum_{k in kb} a*b,
 *     all in FP64 (power-of-two scales make each product exact), blocks in
 *     order; the last K block may be shorter than 128.
 *   - Per-channel scales and bias (DeepGEMM on Hopper, section 5.2: a scale per
 *     channel instead of one per tensor; the bias term of a fused epilogue):
 *     r = sa[m] * sb[n] * acc + bias[n] in FP64 (scale product first, then
 *     the accumulator, then the bias), one BF16 rounding.  A missing scale
 *     vector means 1, a missing bias 0.
 *   - BF16 comparison path (DeepGEMM on Hopper, section 1.3): BF16 operands
 *     (1 sign, 8 exponent, 7 mantissa bits; subnormals decoded), no scales,
 *     D = bf16(sum_k a * b) with the sum in FP64 and one rounding.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_E4M3 0
#define ORACLE_E5M2 1

/* ------------------------------------------------------------------------- */
/* FP8 decode (DeepGEMM on Hopper, section 3.1: the E4M3 / E5M2 bit split).   */
/* ------------------------------------------------------------------------- */

/* Value of one FP8 code, from the sign / exponent / mantissa fields.        */
static double decode_one(int fmt, unsigned code)
{
    unsigned s = (code >> 7) & 1u;
    double sign = s ? -1.0 : 1.0;
    if (fmt == ORACLE_E4M3) {
        unsigned e = (code >> 3) & 0xFu;
        unsigned m = code & 0x7u;
        if (e == 15u && m == 7u) return NAN;                 /* only NaN pattern */
        if (e == 0u) return sign * ldexp((double)m, -9);     /* m/8 * 2^(1-7) */
        return sign * ldexp((double)(8u + m), (int)e - 10);  /* (1+m/8) * 2^(e-7) */
    } else {
        unsigned e = (code >> 2) & 0x1Fu;
        unsigned m = code & 0x3u;
        if (e == 31u) return m ? NAN : sign * INFINITY;
        if (e == 0u) return sign * ldexp((double)m, -16);    /* m/4 * 2^(1-15) */
        return sign * ldexp((double)(4u + m), (int)e - 17);  /* (1+m/4) * 2^(e-15) */
    }
}

int oracle_decode_table(int fmt, double *out256)
{
    if (fmt != ORACLE_E4M3 && fmt != ORACLE_E5M2) return -1;
    for (unsigned c = 0; c < 256u; ++c) out256[c] = decode_one(fmt, c);
    return 0;
}

/* Integer mantissa of each code at the format's finest step: value = n * 2^-q
 * with q = 9 (E4M3) or 16 (E5M2).  Non-finite codes are flagged.             */
static void int_table(int fmt, int64_t *n256, unsigned char *nonfinite256, int *q)
{
    *q = (fmt == ORACLE_E4M3) ? 9 : 16;
    for (unsigned c = 0; c < 256u; ++c) {
        double v = decode_one(fmt, c);
        if (!isfinite(v)) { nonfinite256[c] = 1; n256[c] = 0; continue; }
        nonfinite256[c] = 0;
        n256[c] = (int64_t)ldexp(v, *q);      /* exact: v is a multiple of 2^-q */
    }
}

/* ------------------------------------------------------------------------- */
/* BF16 round-to-nearest-even from a double, in one rounding.                 */
/* ------------------------------------------------------------------------- */
uint16_t oracle_bf16_rne(double x)
{
    if (isnan(x)) return 0x7FC0u;
    uint16_t sign = signbit(x) ? 0x8000u : 0u;
    double a = fabs(x);
    if (isinf(a)) return (uint16_t)(sign | 0x7F80u);
    if (a == 0.0) return sign;
    /* Spacing of BF16 values around a: 2^(e-7) for the binade [2^e, 2^(e+1)),
     * e >= -126; below 2^-126 the subnormal spacing is 2^-133.               */
    int e;
    frexp(a, &e);              /* a = f * 2^e, f in [0.5, 1)  =>  binade e-1 */
    e -= 1;
    if (e < -126) e = -126;
    double ulp = ldexp(1.0, e - 7);
    double q = a / ulp;        /* exact: division by a power of two, q < 2^8 */
    double lo = floor(q);
    double frac = q - lo;      /* exact */
    double n = lo;
    if (frac > 0.5 || (frac == 0.5 && fmod(lo, 2.0) != 0.0)) n = lo + 1.0;
    double r = n * ulp;        /* exact */
    /* Largest finite BF16 is (2 - 2^-7) * 2^127. */
    if (r > ldexp(255.0, 120)) return (uint16_t)(sign | 0x7F80u);
    float f = (float)r;        /* exact: r is a BF16 value */
    uint32_t bits;
    memcpy(&bits, &f, sizeof bits);
    return (uint16_t)(sign | ((bits >> 16) & 0x7FFFu));
}

/* ------------------------------------------------------------------------- */
/* One output element.                                                        */
/* ------------------------------------------------------------------------- */
typedef struct {
    double dec_a[256], dec_b[256];
    int64_t int_a[256], int_b[256];
    unsigned char nf_a[256], nf_b[256];
    int qa, qb;
} tables_t;

static void make_tables(tables_t *t, int a_fmt, int b_fmt)
{
    oracle_decode_table(a_fmt, t->dec_a);
    oracle_decode_table(b_fmt, t->dec_b);
    int_table(a_fmt, t->int_a, t->nf_a, &t->qa);
    int_table(b_fmt, t->int_b, t->nf_b, &t->qb);
}

/* acc = sum_k dec(a[k]) * dec(b[k]) in FP64, in order k = 0..K-1;
 * s   = sum_k |dec(a[k]) * dec(b[k])|;
 * exact (optional): 1 if acc equals the exact integer sum, 0 if it does not,
 * 2 if a non-finite input makes the comparison meaningless.                  */
static void dot(const tables_t *t, const uint8_t *a, const uint8_t *b, int64_t K,
                double *acc_out, double *s_out, unsigned char *exact_out)
{
    double acc = 0.0, s = 0.0;
    for (int64_t k = 0; k < K; ++k) {
        double p = t->dec_a[a[k]] * t->dec_b[b[k]];
        acc += p;
        s += fabs(p);
    }
    *acc_out = acc;
    *s_out = s;
    if (!exact_out) return;
    __int128 isum = 0;
    int nonfinite = 0;
    for (int64_t k = 0; k < K; ++k) {
        if (t->nf_a[a[k]] || t->nf_b[b[k]]) { nonfinite = 1; break; }
        isum += (__int128)t->int_a[a[k]] * (__int128)t->int_b[b[k]];
    }
    if (nonfinite || !isfinite(acc)) { *exact_out = 2; return; }
    /* acc * 2^(qa+qb) must be the integer isum. */
    double scaled = ldexp(acc, t->qa + t->qb);
    if (scaled != floor(scaled) || fabs(scaled) >= ldexp(1.0, 120)) { *exact_out = 0; return; }
    /* Convert scaled to __int128 exactly (|scaled| < 2^120), by magnitude. */
    double mag = fabs(scaled);
    double hi = floor(ldexp(mag, -64));
    double lo = mag - ldexp(hi, 64);        /* exact, 0 <= lo < 2^64 */
    __int128 as_int = ((__int128)(uint64_t)hi << 64) + (__int128)(uint64_t)lo;
    if (scaled < 0) as_int = -as_int;
    *exact_out = (as_int == isum) ? 1 : 0;
}

static void element(const tables_t *t, const uint8_t *arow, const uint8_t *brow, int64_t K,
                    double scale, uint16_t *d, double *r, double *s, unsigned char *ex)
{
    double acc, sabs;
    dot(t, arow, brow, K, &acc, &sabs, ex);
    double rv = acc * scale;
    *d = oracle_bf16_rne(rv);
    if (r) *r = rv;
    if (s) *s = sabs;
}

/* ------------------------------------------------------------------------- */
/* Row-parallel driver: threads split a list of output rows; the arithmetic   */
/* of each element does not depend on the split.                              */
/* ------------------------------------------------------------------------- */
typedef struct {
    const tables_t *t;
    const uint8_t *A, *B;
    int64_t lda, ldb, K, N;
    /* row r of the job: A row a_row[r], B base b_base[r] (rows j*ldb from it),
     * output row out_row[r] (offset into D/R/S in elements), scale[r].        */
    const int64_t *a_row, *b_base, *out_row;
    const double *scale;
    int64_t nrows;
    uint16_t *D; double *R, *S; unsigned char *EX;
    int64_t next;              /* shared work counter (guarded by mu) */
    pthread_mutex_t mu;
} job_t;

static void *worker(void *p)
{
    job_t *j = (job_t *)p;
    for (;;) {
        pthread_mutex_lock(&j->mu);
        int64_t r = j->next++;
        pthread_mutex_unlock(&j->mu);
        if (r >= j->nrows) break;
        const uint8_t *arow = j->A + j->a_row[r] * j->lda;
        const uint8_t *bbase = j->B + j->b_base[r];
        int64_t o = j->out_row[r];
        for (int64_t c = 0; c < j->N; ++c) {
            element(j->t, arow, bbase + c * j->ldb, j->K, j->scale[r],
                    j->D + o + c,
                    j->R ? j->R + o + c : NULL,
                    j->S ? j->S + o + c : NULL,
                    j->EX ? j->EX + o + c : NULL);
        }
    }
    return NULL;
}

static void run_job(job_t *j, int nthreads)
{
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    j->next = 0;
    pthread_mutex_init(&j->mu, NULL);
    pthread_t th[256];
    int started = 0;
    for (int i = 1; i < nthreads; ++i)
        if (pthread_create(&th[started], NULL, worker, j) == 0) ++started;
    worker(j);
    for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
    pthread_mutex_destroy(&j->mu);
}

static int fmt_ok(int f) { return f == ORACLE_E4M3 || f == ORACLE_E5M2; }

/* Dense: D[M x N] (bf16 bits, row stride ldd) = bf16(sa*sb * A[M x K] . B[N x K]^T).
 * R, S, EX (row stride ldd) may be NULL.                                      */
int oracle_gemm_nt(const uint8_t *A, int64_t lda, int a_fmt,
                   const uint8_t *B, int64_t ldb, int b_fmt,
                   float sa, float sb,
                   uint16_t *D, int64_t ldd, double *R, double *S, unsigned char *EX,
                   int64_t M, int64_t N, int64_t K, int nthreads)
{
    if (!fmt_ok(a_fmt) || !fmt_ok(b_fmt) || M < 0 || N < 0 || K < 0) return -1;
    if (M == 0 || N == 0) return 0;
    tables_t *t = (tables_t *)malloc(sizeof *t);
    int64_t *a_row = (int64_t *)malloc(sizeof(int64_t) * M);
    int64_t *b_base = (int64_t *)malloc(sizeof(int64_t) * M);
    int64_t *out_row = (int64_t *)malloc(sizeof(int64_t) * M);
    double *scale = (double *)malloc(sizeof(double) * M);
    if (!t || !a_row || !b_base || !out_row || !scale) {
        free(t); free(a_row); free(b_base); free(out_row); free(scale); return -2;
    }
    make_tables(t, a_fmt, b_fmt);
    double sc = (double)sa * (double)sb;      /* exact in FP64 */
    for (int64_t i = 0; i < M; ++i) {
        a_row[i] = i; b_base[i] = 0; out_row[i] = i * ldd; scale[i] = sc;
    }
    job_t j = {0};
    j.t = t; j.A = A; j.B = B; j.lda = lda; j.ldb = ldb; j.K = K; j.N = N;
    j.a_row = a_row; j.b_base = b_base; j.out_row = out_row; j.scale = scale;
    j.nrows = M; j.D = D; j.R = R; j.S = S; j.EX = EX;
    run_job(&j, nthreads);
    free(t); free(a_row); free(b_base); free(out_row); free(scale);
    return 0;
}

/* Dense, selected elements only: element p is (ii[p], jj[p]).                */
int oracle_gemm_nt_points(const uint8_t *A, int64_t lda, int a_fmt,
                          const uint8_t *B, int64_t ldb, int b_fmt,
                          float sa, float sb, int64_t K,
                          int64_t npts, const int64_t *ii, const int64_t *jj,
                          uint16_t *D, double *R, double *S, unsigned char *EX)
{
    if (!fmt_ok(a_fmt) || !fmt_ok(b_fmt) || K < 0 || npts < 0) return -1;
    tables_t *t = (tables_t *)malloc(sizeof *t);
    if (!t) return -2;
    make_tables(t, a_fmt, b_fmt);
    double sc = (double)sa * (double)sb;
    for (int64_t p = 0; p < npts; ++p)
        element(t, A + ii[p] * lda, B + jj[p] * ldb, K, sc, D + p,
                R ? R + p : NULL, S ? S + p : NULL, EX ? EX + p : NULL);
    free(t);
    return 0;
}

/* Masked grouped: A [G][cap][K], B [G][N][K], D/R/S [G][cap][N].
 * For each g, rows i < clamp(masked_m[g], 0, cap) are computed with scale
 * sa * scale_b[g]; every other row is left as the caller filled it.          */
int oracle_grouped_masked(const uint8_t *A, int a_fmt, const uint8_t *B, int b_fmt,
                          float sa, const float *scale_b, const int32_t *masked_m,
                          uint16_t *D, double *R, double *S, unsigned char *EX,
                          int64_t G, int64_t cap, int64_t N, int64_t K, int nthreads)
{
    if (!fmt_ok(a_fmt) || !fmt_ok(b_fmt) || G < 0 || cap < 0 || N < 0 || K < 0) return -1;
    int64_t total = 0;
    for (int64_t g = 0; g < G; ++g) {
        int64_t m = masked_m[g];
        if (m < 0) m = 0;
        if (m > cap) m = cap;
        total += m;
    }
    if (total == 0 || N == 0) return 0;
    tables_t *t = (tables_t *)malloc(sizeof *t);
    int64_t *a_row = (int64_t *)malloc(sizeof(int64_t) * total);
    int64_t *b_base = (int64_t *)malloc(sizeof(int64_t) * total);
    int64_t *out_row = (int64_t *)malloc(sizeof(int64_t) * total);
    double *scale = (double *)malloc(sizeof(double) * total);
    if (!t || !a_row || !b_base || !out_row || !scale) {
        free(t); free(a_row); free(b_base); free(out_row); free(scale); return -2;
    }
    make_tables(t, a_fmt, b_fmt);
    int64_t r = 0;
    for (int64_t g = 0; g < G; ++g) {
        int64_t m = masked_m[g];
        if (m < 0) m = 0;
        if (m > cap) m = cap;
        for (int64_t i = 0; i < m; ++i, ++r) {
            a_row[r] = g * cap + i;               /* row of the [G*cap][K] view */
            b_base[r] = g * N * K;                /* expert g's weights */
            out_row[r] = (g * cap + i) * N;
            scale[r] = (double)sa * (double)scale_b[g];
        }
    }
    job_t j = {0};
    j.t = t; j.A = A; j.B = B; j.lda = K; j.ldb = K; j.K = K; j.N = N;
    j.a_row = a_row; j.b_base = b_base; j.out_row = out_row; j.scale = scale;
    j.nrows = total; j.D = D; j.R = R; j.S = S; j.EX = EX;
    run_job(&j, nthreads);
    free(t); free(a_row); free(b_base); free(out_row); free(scale);
    return 0;
}

/* Contiguous grouped: A [M_total][K], B [G][N][K], D/R/S [M_total][N].
 * Row r with 0 <= grp_idx[r] < G uses expert grp_idx[r]; other rows are
 * padding and are left as the caller filled them.                            */
int oracle_grouped_contig(const uint8_t *A, int a_fmt, const uint8_t *B, int b_fmt,
                          float sa, const float *scale_b, const int32_t *grp_idx,
                          uint16_t *D, double *R, double *S, unsigned char *EX,
                          int64_t M_total, int64_t G, int64_t N, int64_t K, int nthreads)
{
    if (!fmt_ok(a_fmt) || !fmt_ok(b_fmt) || M_total < 0 || G < 0 || N < 0 || K < 0) return -1;
    int64_t total = 0;
    for (int64_t r = 0; r < M_total; ++r)
        if (grp_idx[r] >= 0 && grp_idx[r] < G) ++total;
    if (total == 0 || N == 0) return 0;
    tables_t *t = (tables_t *)malloc(sizeof *t);
    int64_t *a_row = (int64_t *)malloc(sizeof(int64_t) * total);
    int64_t *b_base = (int64_t *)malloc(sizeof(int64_t) * total);
    int64_t *out_row = (int64_t *)malloc(sizeof(int64_t) * total);
    double *scale = (double *)malloc(sizeof(double) * total);
    if (!t || !a_row || !b_base || !out_row || !scale) {
        free(t); free(a_row); free(b_base); free(out_row); free(scale); return -2;
    }
    make_tables(t, a_fmt, b_fmt);
    int64_t q = 0;
    for (int64_t r = 0; r < M_total; ++r) {
        int32_t g = grp_idx[r];
        if (g < 0 || g >= G) continue;
        a_row[q] = r;
        b_base[q] = (int64_t)g * N * K;
        out_row[q] = r * N;
        scale[q] = (double)sa * (double)scale_b[g];
        ++q;
    }
    job_t j = {0};
    j.t = t; j.A = A; j.B = B; j.lda = K; j.ldb = K; j.K = K; j.N = N;
    j.a_row = a_row; j.b_base = b_base; j.out_row = out_row; j.scale = scale;
    j.nrows = total; j.D = D; j.R = R; j.S = S; j.EX = EX;
    run_job(&j, nthreads);
    free(t); free(a_row); free(b_base); free(out_row); free(scale);
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Block-scaled dense GEMM (UE8M0 scales per 128-element K blocks).           */
/* ------------------------------------------------------------------------- */

/* Value of one unsigned E8M0 scale code.                                     */
static double e8m0_value(uint8_t e)
{
    if (e == 255u) return NAN;
    return ldexp(1.0, (int)e - 127);
}

typedef struct {
    double dec_a[256], dec_b[256];
    const uint8_t *A, *B, *SA, *SB;
    int64_t lda, ldb, lds_a, lds_b, M, N, K;
    uint16_t *D; double *R, *S;
    int64_t ldd;
    int64_t npts; const int64_t *ii, *jj;   /* points mode when ii != NULL */
    int nthreads, tid;
} bs_job_t;

static void bs_element(const bs_job_t *j, int64_t m, int64_t n, uint16_t *d, double *r, double *s)
{
    const uint8_t *a = j->A + m * j->lda;
    const uint8_t *b = j->B + n * j->ldb;
    double acc = 0.0, sabs = 0.0;
    for (int64_t k0 = 0; k0 < j->K; k0 += 128) {
        int64_t k1 = k0 + 128 < j->K ? k0 + 128 : j->K;
        int64_t kb = k0 / 128;
        double part = 0.0, pabs = 0.0;
        for (int64_t k = k0; k < k1; ++k) {
            double p = j->dec_a[a[k]] * j->dec_b[b[k]];
            part += p;
            pabs += fabs(p);
        }
        double sc = e8m0_value(j->SA[kb * j->lds_a + m]) * e8m0_value(j->SB[(n / 128) * j->lds_b + kb]);
        acc += part * sc;
        sabs += pabs * fabs(sc);
    }
    *d = oracle_bf16_rne(acc);
    if (r) *r = acc;
    if (s) *s = sabs;
}

static void *bs_worker(void *p)
{
    bs_job_t *j = (bs_job_t *)p;
    if (j->ii) {
        for (int64_t q = j->tid; q < j->npts; q += j->nthreads)
            bs_element(j, j->ii[q], j->jj[q], j->D + q, j->R ? j->R + q : NULL, j->S ? j->S + q : NULL);
        return NULL;
    }
    for (int64_t m = j->tid; m < j->M; m += j->nthreads)
        for (int64_t n = 0; n < j->N; ++n) {
            int64_t o = m * j->ldd + n;
            bs_element(j, m, n, j->D + o, j->R ? j->R + o : NULL, j->S ? j->S + o : NULL);
        }
    return NULL;
}

static int bs_run(bs_job_t *base, int a_fmt, int b_fmt, int nthreads)
{
    oracle_decode_table(a_fmt, base->dec_a);
    oracle_decode_table(b_fmt, base->dec_b);
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    bs_job_t *jobs = (bs_job_t *)malloc(sizeof(bs_job_t) * (size_t)nthreads);
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    if (!jobs || !th) { free(jobs); free(th); return -2; }
    int started = 0;
    for (int i = 0; i < nthreads; ++i) {
        jobs[i] = *base;
        jobs[i].nthreads = nthreads;
        jobs[i].tid = i;
    }
    for (int i = 1; i < nthreads; ++i)
        if (pthread_create(&th[i], NULL, bs_worker, &jobs[i]) == 0) ++started;
        else { jobs[i].tid = -1; }
    bs_worker(&jobs[0]);
    for (int i = 1; i < nthreads; ++i)
        if (jobs[i].tid >= 0) pthread_join(th[i], NULL);
    /* a thread that failed to start: do its share here */
    for (int i = 1; i < nthreads; ++i)
        if (jobs[i].tid < 0) { jobs[i].tid = i; bs_worker(&jobs[i]); }
    free(jobs); free(th);
    (void)started;
    return 0;
}

/* Block-scaled dense: D[M x N] (bf16 bits, row stride ldd).
 *   scale_a: E8M0 codes, scale of (row m, K block kb) at scale_a[kb * lds_a + m]
 *   scale_b: E8M0 codes, scale of (rows 128 nb .. 128 nb + 127, K block kb) at
 *            scale_b[nb * lds_b + kb]
 * R and S (row stride ldd) may be NULL; S is sum_k |a b| * scale.            */
int oracle_gemm_nt_blockscaled(const uint8_t *A, int64_t lda, int a_fmt,
                               const uint8_t *B, int64_t ldb, int b_fmt,
                               const uint8_t *scale_a, int64_t lds_a,
                               const uint8_t *scale_b, int64_t lds_b,
                               uint16_t *D, int64_t ldd, double *R, double *S,
                               int64_t M, int64_t N, int64_t K, int nthreads)
{
    if (!fmt_ok(a_fmt) || !fmt_ok(b_fmt) || M < 0 || N < 0 || K < 0) return -1;
    if (M == 0 || N == 0) return 0;
    bs_job_t j;
    memset(&j, 0, sizeof j);
    j.A = A; j.B = B; j.SA = scale_a; j.SB = scale_b;
    j.lda = lda; j.ldb = ldb; j.lds_a = lds_a; j.lds_b = lds_b;
    j.M = M; j.N = N; j.K = K; j.D = D; j.R = R; j.S = S; j.ldd = ldd;
    return bs_run(&j, a_fmt, b_fmt, nthreads);
}

/* Block-scaled dense, selected elements (ii[p], jj[p]) only.                 */
int oracle_gemm_nt_blockscaled_points(const uint8_t *A, int64_t lda, int a_fmt,
                                      const uint8_t *B, int64_t ldb, int b_fmt,
                                      const uint8_t *scale_a, int64_t lds_a,
                                      const uint8_t *scale_b, int64_t lds_b, int64_t K,
                                      int64_t npts, const int64_t *ii, const int64_t *jj,
                                      uint16_t *D, double *R, double *S, int nthreads)
{
    if (!fmt_ok(a_fmt) || !fmt_ok(b_fmt) || K < 0 || npts < 0) return -1;
    if (npts == 0) return 0;
    bs_job_t j;
    memset(&j, 0, sizeof j);
    j.A = A; j.B = B; j.SA = scale_a; j.SB = scale_b;
    j.lda = lda; j.ldb = ldb; j.lds_a = lds_a; j.lds_b = lds_b;
    j.K = K; j.D = D; j.R = R; j.S = S; j.npts = npts; j.ii = ii; j.jj = jj;
    return bs_run(&j, a_fmt, b_fmt, nthreads);
}

/* ------------------------------------------------------------------------- */
/* Dense GEMM with per-row / per-channel scales and a per-channel bias.       */
/* ------------------------------------------------------------------------- */

/* D[M x N] (bf16 bits, row stride ldd) = bf16(sa[m] * sb[n] * A[m] . B[n] + bias[n]).
 * scale_a [M], scale_b [N], bias [N] may each be NULL (1, 1, 0).  R and S
 * (row stride ldd) may be NULL; S = sum_k |a b| * |sa[m] * sb[n]|.           */
int oracle_gemm_nt_channelwise(const uint8_t *A, int64_t lda, int a_fmt,
                               const uint8_t *B, int64_t ldb, int b_fmt,
                               const float *scale_a, const float *scale_b, const float *bias,
                               uint16_t *D, int64_t ldd, double *R, double *S,
                               int64_t M, int64_t N, int64_t K)
{
    if (!fmt_ok(a_fmt) || !fmt_ok(b_fmt) || M < 0 || N < 0 || K < 0) return -1;
    if (M == 0 || N == 0) return 0;
    tables_t *t = (tables_t *)malloc(sizeof *t);
    if (!t) return -2;
    make_tables(t, a_fmt, b_fmt);
    for (int64_t m = 0; m < M; ++m) {
        double sam = scale_a ? (double)scale_a[m] : 1.0;
        for (int64_t n = 0; n < N; ++n) {
            double acc, sabs;
            dot(t, A + m * lda, B + n * ldb, K, &acc, &sabs, NULL);
            double sc = sam * (scale_b ? (double)scale_b[n] : 1.0);
            double r = sc * acc + (bias ? (double)bias[n] : 0.0);
            D[m * ldd + n] = oracle_bf16_rne(r);
            if (R) R[m * ldd + n] = r;
            if (S) S[m * ldd + n] = sabs * fabs(sc);
        }
    }
    free(t);
    return 0;
}

/* Block-scaled masked grouped: A [G][cap][K], B [G][N][K], D/R/S [G][cap][N];
 * scale_a [G][ceil(K/128)][lds_a] (row m of group g over K block kb at
 * g * KB * lds_a + kb * lds_a + m), scale_b [G][ceil(N/128)][lds_b].  Rows
 * i < clamp(masked_m[g], 0, cap) are computed; the others are left as the
 * caller filled them.                                                        */
int oracle_grouped_masked_blockscaled(const uint8_t *A, int a_fmt, const uint8_t *B, int b_fmt,
                                      const uint8_t *scale_a, int64_t lds_a,
                                      const uint8_t *scale_b, int64_t lds_b, const int32_t *masked_m,
                                      uint16_t *D, double *R, double *S,
                                      int64_t G, int64_t cap, int64_t N, int64_t K, int nthreads)
{
    if (!fmt_ok(a_fmt) || !fmt_ok(b_fmt) || G < 0 || cap < 0 || N < 0 || K < 0) return -1;
    int64_t kb = (K + 127) / 128, nb = (N + 127) / 128;
    for (int64_t g = 0; g < G; ++g) {
        int64_t mg = masked_m[g];
        if (mg < 0) mg = 0;
        if (mg > cap) mg = cap;
        if (mg == 0 || N == 0) continue;
        int rc = oracle_gemm_nt_blockscaled(A + g * cap * K, K, a_fmt, B + g * N * K, K, b_fmt,
                                            scale_a + g * kb * lds_a, lds_a, scale_b + g * nb * lds_b, lds_b,
                                            D + g * cap * N, N, R ? R + g * cap * N : NULL,
                                            S ? S + g * cap * N : NULL, mg, N, K, nthreads);
        if (rc != 0) return rc;
    }
    return 0;
}

/* Block-scaled contiguous grouped: A [M_total][K], B [G][N][K], D/R/S [M_total][N];
 * scale_a [ceil(K/128)][lds_a] (row r over K block kb at kb * lds_a + r, r the
 * global row), scale_b [G][ceil(N/128)][lds_b].  Row r with 0 <= grp_idx[r] < G
 * uses expert grp_idx[r]; other rows are padding and are left untouched.    */
int oracle_grouped_contig_blockscaled(const uint8_t *A, int a_fmt, const uint8_t *B, int b_fmt,
                                      const uint8_t *scale_a, int64_t lds_a,
                                      const uint8_t *scale_b, int64_t lds_b, const int32_t *grp_idx,
                                      uint16_t *D, double *R, double *S,
                                      int64_t M_total, int64_t G, int64_t N, int64_t K)
{
    if (!fmt_ok(a_fmt) || !fmt_ok(b_fmt) || M_total < 0 || G < 0 || N < 0 || K < 0) return -1;
    int64_t kb = (K + 127) / 128, nb = (N + 127) / 128;
    for (int64_t r = 0; r < M_total; ++r) {
        int32_t e = grp_idx[r];
        if (e < 0 || e >= G || N == 0) continue;
        /* one row: the dense block-scaled form with the row's scale column */
        uint8_t *col = (uint8_t *)malloc((size_t)(kb > 0 ? kb : 1));
        if (!col) return -2;
        for (int64_t b = 0; b < kb; ++b) col[b] = scale_a[b * lds_a + r];
        int rc = oracle_gemm_nt_blockscaled(A + r * K, K, a_fmt, B + e * N * K, K, b_fmt, col, 1,
                                            scale_b + e * nb * lds_b, lds_b, D + r * N, N,
                                            R ? R + r * N : NULL, S ? S + r * N : NULL, 1, N, K, 1);
        free(col);
        if (rc != 0) return rc;
    }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* BF16 comparison path (DeepGEMM on Hopper, section 1.3: the backend keeps a */
/* BF16 path for precision experiments).  Reading: D = bf16(A . B^T) with     */
/* BF16 operands, no scales, the product sum in FP64 in order k = 0..K-1 and  */
/* one BF16 rounding, exactly as the FP8 forms do after decoding.             */
/* ------------------------------------------------------------------------- */

/* Value of one BF16 bit pattern from its fields: sign, 8 exponent bits (bias
 * 127), 7 mantissa bits; exponent 0 is zero / subnormal (m * 2^-133),
 * exponent 255 is infinity (m = 0) or NaN.                                   */
double oracle_bf16_value(uint16_t bits)
{
    int sign = (bits >> 15) & 1;
    int e = (bits >> 7) & 0xFF;
    int m = bits & 0x7F;
    double v;
    if (e == 0xFF) v = m ? NAN : INFINITY;
    else if (e == 0) v = ldexp((double)m, -133);
    else v = ldexp(128.0 + (double)m, e - 127 - 7);
    return sign ? -v : v;
}

static void dot_bf16(const uint16_t *a, const uint16_t *b, int64_t K, double *acc_out, double *s_out)
{
    double acc = 0.0, s = 0.0;
    for (int64_t k = 0; k < K; ++k) {
        double p = oracle_bf16_value(a[k]) * oracle_bf16_value(b[k]);   /* exact: 8 x 8 significant bits */
        acc += p;
        s += fabs(p);
    }
    *acc_out = acc;
    *s_out = s;
}

/* A [M][lda], B [N][ldb] BF16 bit patterns (K-contiguous rows); D [M][ldd]
 * BF16 bits; R (the FP64 sum) and S (sum of |products|) optional, [M][ldd]. */
int oracle_gemm_nt_bf16(const uint16_t *A, int64_t lda, const uint16_t *B, int64_t ldb,
                        uint16_t *D, int64_t ldd, double *R, double *S,
                        int64_t M, int64_t N, int64_t K)
{
    if (M < 0 || N < 0 || K < 0 || lda < K || ldb < K || ldd < N) return -1;
    for (int64_t i = 0; i < M; ++i)
        for (int64_t j = 0; j < N; ++j) {
            double acc, sabs;
            dot_bf16(A + i * lda, B + j * ldb, K, &acc, &sabs);
            D[i * ldd + j] = oracle_bf16_rne(acc);
            if (R) R[i * ldd + j] = acc;
            if (S) S[i * ldd + j] = sabs;
        }
    return 0;
}

/* The same at selected elements (ii[p], jj[p]) only; D, R, S have npts entries. */
int oracle_gemm_nt_bf16_points(const uint16_t *A, int64_t lda, const uint16_t *B, int64_t ldb, int64_t K,
                               int64_t npts, const int64_t *ii, const int64_t *jj,
                               uint16_t *D, double *R, double *S)
{
    if (K < 0 || npts < 0 || lda < K || ldb < K) return -1;
    for (int64_t p = 0; p < npts; ++p) {
        double acc, sabs;
        dot_bf16(A + ii[p] * lda, B + jj[p] * ldb, K, &acc, &sabs);
        D[p] = oracle_bf16_rne(acc);
        if (R) R[p] = acc;
        if (S) S[p] = sabs;
    }
    return 0;
}
