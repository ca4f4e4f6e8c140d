/*
 * frn_oracle.c -- plain, slow CPU oracle of the fused reduce + norm boundary.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke check in
 * __graft_entry__.py and the CPU-baseline leg of bench.py may load this
 * library.  The GPU library shares no source, header, table or helper with
 * it, and neither one includes, links or calls the other.
 *
 * What is computed, and where it is defined:
 *
 *   vLLM PR #62366 (Beam fused all-reduce + sandwich norms + top-k finalize),
 *   sections "Overview" and "Claims": a TP all-reduce of BF16 partial sums in
 *   FP32, followed either by residual add + RMSNorm or by Beam's FP32
 *   norm -> residual add -> norm epilogue, with an optional MoE top-k
 *   finalize done on each rank, and rounded to BF16 there, before the
 *   reduction.  For large batches the reduction alone produces a BF16 tensor
 *   and a separate boundary kernel runs the epilogue on it.
 *   Section "Details": the FP32 boundary math is built without FMA
 *   contraction.
 *
 *   SGLang PR #34134 (FlashInfer CuTe-DSL MNNVL fusion backend), first commit
 *   message: the two fused patterns, all-reduce + residual + RMSNorm, and MoE
 *   finalize + shared-expert add + all-reduce + residual + RMSNorm.
 *
 * The pages fix FP32 arithmetic and BF16 storage but never write a formula
 * or an operation order.  This file takes one plain order and sticks to it:
 *
 *   finalize   acc = +0; for j = 0..k-1: acc = acc + (w[t,j] * E[idx[t,j],i]);
 *              then acc = acc + S[t,i] when a shared expert is given;
 *              P = bf16(acc).  Each * and + is one rounded FP32 operation.
 *   reduce     s = P_0; for r = 1..R-1: s = s + P_r   (FP32, r ascending).
 *   inv_rms    ss = sum_i x_i^2, squares exact in FP64, summed in FP64 with i
 *              ascending; ms = (float)(ss / H); v = ms + eps; d = sqrtf(v);
 *              rinv = 1 / d  (each step one correctly rounded FP32 op).
 *   rmsnorm    h = s + x; xout = bf16(h); r = inv_rms(h);
 *              y = bf16((h * r) * gamma).
 *   sandwich   r1 = inv_rms(s); a = (s * r1) * gamma1; h = a + x;
 *              xout = bf16(h); r2 = inv_rms(h); y = bf16((h * r2) * gamma2).
 *   split      U = bf16(s) (pass 1), then rmsnorm / sandwich with R = 1 on U.
 *
 *   expert-parallel finalize (vLLM PR #62366 "Overview" and "Details": the
 *   replicated-token deferral for TP = 1, EP > 1 that builds on the same
 *   fused boundary):  every rank holds all T tokens and the same weights
 *   w[t,j], but expert rows only for its own experts.  idx_r[t,j] is the row
 *   of rank r's buffer for slot j, or negative when slot j's expert lives on
 *   another rank.  Rank r's finalize is the one above over its own slots
 *   only, j ascending, plus its shared-expert row if it holds one; the R
 *   BF16 partials then go through the same reduce and epilogue.
 *
 * bf16(f) rounds binary32 to bfloat16, nearest with ties to even; NaN stays a
 * quiet NaN with its sign, overflow goes to +-inf.  Widening is exact.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off (no fast-math), so that every
 * FP32 operation above is one IEEE operation.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef uint16_t bf16_t;

/* ---------------------------------------------------------------- BF16 --- */

float oracle_bf16_to_f32(bf16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

bf16_t oracle_f32_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7fffffffu) > 0x7f800000u) /* NaN: keep sign, force quiet bit */
        return (bf16_t)((u >> 16) | 0x0040u);
    /* Round to nearest, ties to even, on the 16 bits that are dropped. */
    uint32_t upper = u >> 16;
    uint32_t lower = u & 0xffffu;
    if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u)))
        upper += 1u; /* carries into the exponent; 0x7f7f.. rounds to inf */
    return (bf16_t)upper;
}

void oracle_bf16_to_f32_array(const bf16_t* in, float* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_bf16_to_f32(in[i]);
}

void oracle_f32_to_bf16_array(const float* in, bf16_t* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f32_to_bf16(in[i]);
}

/* ------------------------------------------------------- method steps --- */

/*
 * MoE top-k finalize for one token row of one rank (vLLM #62366 "Claims";
 * SGLang #34134 second fusion pattern).  rows is that rank's expert output
 * buffer [num_rows, H]; idx/w are the token's k slots; shared is that rank's
 * shared-expert row or NULL.  An index outside [0, num_rows) is never
 * dereferenced: its slot reads as NaN, so the whole row turns NaN.
 */
static void finalize_row(const bf16_t* rows, int64_t num_rows,
                         const bf16_t* shared_row, const float* w,
                         const int32_t* idx, int32_t k, int64_t H,
                         bf16_t* p_row)
{
    for (int64_t i = 0; i < H; ++i) {
        float acc = 0.0f;
        for (int32_t j = 0; j < k; ++j) {
            float e;
            if (idx[j] < 0 || (int64_t)idx[j] >= num_rows)
                e = NAN;
            else
                e = oracle_bf16_to_f32(rows[(int64_t)idx[j] * H + i]);
            float prod = w[j] * e;
            acc = acc + prod;
        }
        if (shared_row) acc = acc + oracle_bf16_to_f32(shared_row[i]);
        p_row[i] = oracle_f32_to_bf16(acc);
    }
}

/*
 * Expert-parallel finalize of one token row of rank r: the slots whose idx
 * is negative belong to another rank's experts and take no part in this
 * rank's sum (they are skipped, not added as zero).  An index at or past
 * num_rows reads as NaN, as above.  shared_row is NULL when this rank holds
 * no shared-expert row.
 */
static void finalize_row_ep(const bf16_t* rows, int64_t num_rows,
                            const bf16_t* shared_row, const float* w,
                            const int32_t* idx, int32_t k, int64_t H,
                            bf16_t* p_row)
{
    for (int64_t i = 0; i < H; ++i) {
        float acc = 0.0f;
        for (int32_t j = 0; j < k; ++j) {
            if (idx[j] < 0) continue; /* another rank's expert */
            float e;
            if ((int64_t)idx[j] >= num_rows)
                e = (float)NAN;
            else
                e = oracle_bf16_to_f32(rows[(int64_t)idx[j] * H + i]);
            float term = w[j] * e;
            acc = acc + term;
        }
        if (shared_row != NULL) acc = acc + oracle_bf16_to_f32(shared_row[i]);
        p_row[i] = oracle_f32_to_bf16(acc);
    }
}

/* Step a: FP32 sum over the R partials, r ascending, for one row. */
static void reduce_row(const bf16_t* const* p_rows, int32_t R, int64_t H,
                       float* s)
{
    for (int64_t i = 0; i < H; ++i) {
        float acc = oracle_bf16_to_f32(p_rows[0][i]);
        for (int32_t r = 1; r < R; ++r)
            acc = acc + oracle_bf16_to_f32(p_rows[r][i]);
        s[i] = acc;
    }
}

/* Inverse RMS of one FP32 row, eps inside the root (standard RMSNorm). */
float oracle_inv_rms(const float* x, int64_t H, float eps, double* ss_out)
{
    double ss = 0.0;
    for (int64_t i = 0; i < H; ++i) {
        double xi = (double)x[i];
        double sq = xi * xi; /* exact: 24-bit mantissa squared fits 53 bits */
        ss = ss + sq;
    }
    if (ss_out) *ss_out = ss;
    float ms = (float)(ss / (double)H);
    float v = ms + eps;
    float d = sqrtf(v);
    return 1.0f / d;
}

/* Debug outputs (any pointer may be NULL).  Row-major [T,H] or [T]. */
typedef struct {
    float* s;    /* FP32 reduced sum                       */
    float* a;    /* sandwich: first-norm output (s*r1)*g1  */
    float* h;    /* FP32 value stored to the new residual  */
    float* y;    /* FP32 normed output before BF16 rounding */
    float* r1;   /* inverse RMS of s (sandwich) or of h (rmsnorm) */
    float* r2;   /* inverse RMS of h (sandwich only)        */
    double* ss1; /* FP64 sum of squares behind r1           */
    double* ss2; /* FP64 sum of squares behind r2           */
    bf16_t* p;   /* [R,T,H] finalized partials (finalize only) */
    bf16_t* u;   /* [T,H] split pass-1 output                */
} oracle_debug;

enum { ORACLE_EPI_RMSNORM = 0, ORACLE_EPI_SANDWICH = 1, ORACLE_EPI_NONE = 2 };

/* Residual add + RMSNorm on one row (vLLM #62366 microbenchmark table;
 * SGLang #34134 first pattern). */
static void rmsnorm_row(const float* s, const bf16_t* x, const float* gamma,
                        float eps, int64_t H, float* h, bf16_t* y,
                        bf16_t* xout, float* y32, float* r_out,
                        double* ss_out)
{
    for (int64_t i = 0; i < H; ++i) {
        h[i] = s[i] + oracle_bf16_to_f32(x[i]);
        xout[i] = oracle_f32_to_bf16(h[i]);
    }
    float r = oracle_inv_rms(h, H, eps, ss_out);
    if (r_out) *r_out = r;
    for (int64_t i = 0; i < H; ++i) {
        float n = h[i] * r;
        float o = n * gamma[i];
        if (y32) y32[i] = o;
        y[i] = oracle_f32_to_bf16(o);
    }
}

/* Beam's FP32 norm -> residual add -> norm (vLLM #62366 "Overview",
 * "Claims"). */
static void sandwich_row(const float* s, const bf16_t* x, const float* g1,
                         const float* g2, float eps, int64_t H, float* a,
                         float* h, bf16_t* y, bf16_t* xout, float* y32,
                         float* r1_out, float* r2_out, double* ss1_out,
                         double* ss2_out)
{
    float r1 = oracle_inv_rms(s, H, eps, ss1_out);
    if (r1_out) *r1_out = r1;
    for (int64_t i = 0; i < H; ++i) {
        float n = s[i] * r1;
        a[i] = n * g1[i];
        h[i] = a[i] + oracle_bf16_to_f32(x[i]);
        xout[i] = oracle_f32_to_bf16(h[i]);
    }
    float r2 = oracle_inv_rms(h, H, eps, ss2_out);
    if (r2_out) *r2_out = r2;
    for (int64_t i = 0; i < H; ++i) {
        float n = h[i] * r2;
        float o = n * g2[i];
        if (y32) y32[i] = o;
        y[i] = oracle_f32_to_bf16(o);
    }
}

/* ------------------------------------------------------ whole boundary --- */

typedef struct {
    /* partials (k == 0) or expert rows (k > 0): R pointers */
    const bf16_t* const* src;
    const bf16_t* const* shared; /* R pointers or NULL (finalize only) */
    int32_t R;
    const float* w;     /* [T,k] */
    const int32_t* idx; /* [T,k] */
    int32_t k;          /* 0: no finalize */
    int64_t num_rows;
    /* expert-parallel finalize: R index arrays [T,k] and R row counts */
    const int32_t* const* idx_r;
    const int64_t* num_rows_r;
    int32_t epilogue;   /* ORACLE_EPI_* */
    int32_t split;      /* 1: round s to BF16 and restart with R = 1 */
    const bf16_t* x;    /* residual in [T,H] */
    const float* g1;
    const float* g2;
    float eps;
    int64_t T, H;
    bf16_t* y;          /* [T,H] (epilogue != NONE) */
    bf16_t* xout;       /* [T,H] (epilogue != NONE) */
    bf16_t* u;          /* [T,H] reduced sum in BF16 (epilogue == NONE) */
    const oracle_debug* dbg;
} job_t;

typedef struct {
    const job_t* job;
    int64_t t0, t1;
    int status;
} slice_t;

static float* dbg_row(float* base, int64_t t, int64_t H)
{
    return base ? base + t * H : NULL;
}

static void* run_rows(void* arg)
{
    slice_t* sl = (slice_t*)arg;
    const job_t* J = sl->job;
    const oracle_debug* D = J->dbg;
    const int64_t H = J->H;
    float* s = malloc(sizeof(float) * (size_t)H);
    float* a = malloc(sizeof(float) * (size_t)H);
    float* h = malloc(sizeof(float) * (size_t)H);
    bf16_t* p = J->k > 0 ? malloc(sizeof(bf16_t) * (size_t)H * (size_t)J->R) : NULL;
    bf16_t* u = malloc(sizeof(bf16_t) * (size_t)H);
    const bf16_t** rows = malloc(sizeof(bf16_t*) * (size_t)J->R);
    if (!s || !a || !h || !u || !rows || (J->k > 0 && !p)) {
        sl->status = -1;
        goto out;
    }
    for (int64_t t = sl->t0; t < sl->t1; ++t) {
        /* optional finalize, one rank at a time, into BF16 rows */
        for (int32_t r = 0; r < J->R; ++r) {
            if (J->k > 0 && J->idx_r) {
                finalize_row_ep(J->src[r], J->num_rows_r[r],
                                J->shared && J->shared[r] ? J->shared[r] + t * H : NULL,
                                J->w + t * J->k, J->idx_r[r] + t * J->k, J->k, H,
                                p + (int64_t)r * H);
                rows[r] = p + (int64_t)r * H;
                if (D && D->p)
                    memcpy(D->p + ((int64_t)r * J->T + t) * H, rows[r],
                           sizeof(bf16_t) * (size_t)H);
            } else if (J->k > 0) {
                finalize_row(J->src[r], J->num_rows,
                             J->shared ? J->shared[r] + t * H : NULL,
                             J->w + t * J->k, J->idx + t * J->k, J->k, H,
                             p + (int64_t)r * H);
                rows[r] = p + (int64_t)r * H;
                if (D && D->p)
                    memcpy(D->p + ((int64_t)r * J->T + t) * H, rows[r],
                           sizeof(bf16_t) * (size_t)H);
            } else {
                rows[r] = J->src[r] + t * H;
            }
        }
        reduce_row(rows, J->R, H, s);
        if (J->split || J->epilogue == ORACLE_EPI_NONE) {
            /* large-batch path: the reduction's output is a BF16 tensor */
            for (int64_t i = 0; i < H; ++i) u[i] = oracle_f32_to_bf16(s[i]);
            if (D && D->u) memcpy(D->u + t * H, u, sizeof(bf16_t) * (size_t)H);
            if (J->epilogue == ORACLE_EPI_NONE) {
                memcpy(J->u + t * H, u, sizeof(bf16_t) * (size_t)H);
                if (D && D->s) memcpy(D->s + t * H, s, sizeof(float) * (size_t)H);
                continue;
            }
            const bf16_t* one[1] = {u};
            reduce_row(one, 1, H, s); /* pass 2 starts from U with R = 1 */
        }
        if (D && D->s) memcpy(D->s + t * H, s, sizeof(float) * (size_t)H);
        float r1 = 0.0f, r2 = 0.0f;
        double ss1 = 0.0, ss2 = 0.0;
        if (J->epilogue == ORACLE_EPI_RMSNORM) {
            rmsnorm_row(s, J->x + t * H, J->g1, J->eps, H, h, J->y + t * H,
                        J->xout + t * H, D ? dbg_row(D->y, t, H) : NULL, &r1,
                        &ss1);
        } else {
            sandwich_row(s, J->x + t * H, J->g1, J->g2, J->eps, H, a, h,
                         J->y + t * H, J->xout + t * H,
                         D ? dbg_row(D->y, t, H) : NULL, &r1, &r2, &ss1, &ss2);
            if (D && D->a) memcpy(D->a + t * H, a, sizeof(float) * (size_t)H);
            if (D && D->r2) D->r2[t] = r2;
            if (D && D->ss2) D->ss2[t] = ss2;
        }
        if (D && D->h) memcpy(D->h + t * H, h, sizeof(float) * (size_t)H);
        if (D && D->r1) D->r1[t] = r1;
        if (D && D->ss1) D->ss1[t] = ss1;
    }
    sl->status = 0;
out:
    free(s);
    free(a);
    free(h);
    free(p);
    free(u);
    free(rows);
    return NULL;
}

/* Rows are independent, so the split over threads cannot change a result. */
static int run_job(const job_t* J, int32_t nthreads)
{
    if (J->T <= 0) return 0;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > J->T) nthreads = (int32_t)J->T;
    slice_t* sl = calloc((size_t)nthreads, sizeof(slice_t));
    pthread_t* th = calloc((size_t)nthreads, sizeof(pthread_t));
    if (!sl || !th) {
        free(sl);
        free(th);
        return -1;
    }
    int rc = 0;
    for (int32_t i = 0; i < nthreads; ++i) {
        sl[i].job = J;
        sl[i].t0 = J->T * i / nthreads;
        sl[i].t1 = J->T * (i + 1) / nthreads;
        sl[i].status = -1;
    }
    if (nthreads == 1) {
        run_rows(&sl[0]);
    } else {
        for (int32_t i = 0; i < nthreads; ++i)
            if (pthread_create(&th[i], NULL, run_rows, &sl[i]) != 0) {
                run_rows(&sl[i]);
                th[i] = 0;
            }
        for (int32_t i = 0; i < nthreads; ++i)
            if (th[i]) pthread_join(th[i], NULL);
    }
    for (int32_t i = 0; i < nthreads; ++i)
        if (sl[i].status != 0) rc = -1;
    free(sl);
    free(th);
    return rc;
}

/*
 * The whole boundary on the CPU.  k == 0: src holds the R BF16 partials
 * [T,H].  k > 0: src holds the R expert-row buffers [num_rows,H]; w/idx are
 * [T,k]; shared is NULL or R shared-expert buffers [T,H].  epilogue selects
 * residual + RMSNorm (g1 = gamma), the sandwich (g1, g2), or none (reduction
 * only, output u).  split = 1 rounds the reduced sum to BF16 and runs the
 * epilogue from that tensor (the large-batch two-pass path).
 * Returns 0 on success, -1 on bad arguments or allocation failure.
 */
int oracle_boundary(const bf16_t* const* src, const bf16_t* const* shared,
                    int32_t R, const float* w, const int32_t* idx, int32_t k,
                    int64_t num_rows, int32_t epilogue, int32_t split,
                    const bf16_t* x, const float* g1, const float* g2,
                    float eps, int64_t T, int64_t H, bf16_t* y, bf16_t* xout,
                    bf16_t* u, const oracle_debug* dbg, int32_t nthreads)
{
    if (R < 1 || k < 0 || T < 0 || H < 1 || !src) return -1;
    if (epilogue < ORACLE_EPI_RMSNORM || epilogue > ORACLE_EPI_NONE) return -1;
    if (k > 0 && (!w || !idx)) return -1;
    if (epilogue != ORACLE_EPI_NONE && (!x || !g1 || !y || !xout)) return -1;
    if (epilogue == ORACLE_EPI_SANDWICH && !g2) return -1;
    if (epilogue == ORACLE_EPI_NONE && !u) return -1;
    job_t J = {src, shared, R, w, idx, k, num_rows, NULL, NULL, epilogue, split,
               x, g1, g2, eps, T, H, y, xout, u, dbg};
    return run_job(&J, nthreads);
}

/*
 * The boundary with the expert-parallel finalize (see the header of this
 * file).  src holds R expert-row buffers, src[r] of num_rows_r[r] rows
 * (NULL allowed when that count is 0); idx_r holds R index arrays [T,k];
 * w is [T,k], the same for every rank; shared is NULL, or R pointers of
 * which any may be NULL (that rank holds no shared-expert row).  The other
 * arguments are those of oracle_boundary.
 */
int oracle_ep_boundary(const bf16_t* const* src, const bf16_t* const* shared,
                       int32_t R, const float* w, const int32_t* const* idx_r,
                       int32_t k, const int64_t* num_rows_r, int32_t epilogue,
                       int32_t split, const bf16_t* x, const float* g1,
                       const float* g2, float eps, int64_t T, int64_t H,
                       bf16_t* y, bf16_t* xout, bf16_t* u,
                       const oracle_debug* dbg, int32_t nthreads)
{
    if (R < 1 || k < 1 || T < 0 || H < 1 || !src || !w || !idx_r || !num_rows_r)
        return -1;
    if (epilogue < ORACLE_EPI_RMSNORM || epilogue > ORACLE_EPI_NONE) return -1;
    if (epilogue != ORACLE_EPI_NONE && (!x || !g1 || !y || !xout)) return -1;
    if (epilogue == ORACLE_EPI_SANDWICH && !g2) return -1;
    if (epilogue == ORACLE_EPI_NONE && !u) return -1;
    for (int32_t r = 0; r < R; ++r) {
        if (!idx_r[r] || num_rows_r[r] < 0) return -1;
        if (num_rows_r[r] > 0 && !src[r]) return -1;
    }
    job_t J = {src, shared, R, w, NULL, k, 0, idx_r, num_rows_r, epilogue, split,
               x, g1, g2, eps, T, H, y, xout, u, dbg};
    return run_job(&J, nthreads);
}
