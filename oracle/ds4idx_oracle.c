/*
 * CPU oracle for the Lightning Indexer: score every causally visible cached key
 * for each query token, keep the top-k positions.
 *
 * TEST INFRASTRUCTURE. This file is the plain, slow reference that the HIP path
 * is checked against. Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg may build, load or call it. It shares no code, header, table
 * or helper with the HIP library, and the HIP library never calls it.
 *
 * What it computes (the plain definition, written out):
 *
 *   The Lightning Indexer sits in DeepSeek V4's sparse attention and, for every
 *   query token, picks the positions of the long context worth attending to;
 *   its two stages are a scorer and a top-512 selection (first page,
 *   "DeepSeek V4 Flash 추론을 1.6초로 줄인 ds4 최적화", glossary entry
 *   "Lightning Indexer" and section details, second paragraph). The pages name
 *   the scorer but do not print its formula; the formula used is the indexer's
 *   published scoring form
 *
 *       score(t, s) = sum_h  w[t,h] * max(0, sum_d q[t,h,d] * k[s,d])
 *
 *   over the H indexer heads, with query t (absolute position offset + t)
 *   seeing cached keys s <= offset + t.  Selection keeps the min(k, L) visible
 *   keys that come first in the order (score descending, index ascending), a
 *   strict total order, so the answer is unique; equal scores go to the lower
 *   index.  The ds4 kernel changes left every logit byte-identical (first
 *   page, TL;DR and section details), i.e. the selection is an exact function
 *   of its inputs, not an approximation.
 *
 *   Output: the selected indices in ascending order, padded with -1 up to k.
 *
 * Arithmetic: every input is decoded to double exactly (fp32, bf16, and OCP
 * E4M3 codes times an fp32 per-token scale: a 4-bit by 24-bit significand
 * product fits a double), products q*k are exact in double (<= 36 significant
 * bits), sums are accumulated in double in index order.  -0.0 and +0.0 compare
 * equal (plain IEEE comparisons), so a row of zeros falls to the index rule.
 *
 * FP8: OCP E4M3FN (sign, 4 exponent bits with bias 7, 3 mantissa bits;
 * exponent 0 is subnormal; S.1111.111 is NaN; no infinities; max 448).  The
 * MI300X write-up ("DeepSeek V4 Flash는 단일 AMD MI300X에서 실행됩니다",
 * section on the FP8 format mismatch) records what goes wrong when the same
 * bits are read as the FNUZ variant (bias 8): a 2x scale error. This decoder
 * is OCP only.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { O_F32 = 0, O_BF16 = 1, O_FP8 = 2, O_F64 = 3 };

/* OCP E4M3FN code -> exact value. */
double ds4o_e4m3_decode(int code)
{
    int sign = (code >> 7) & 1;
    int e = (code >> 3) & 15;
    int m = code & 7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);          /* (m / 8) * 2^(1 - 7) */
    else
        v = ldexp((double)(8 + m), e - 10); /* (1 + m / 8) * 2^(e - 7) */
    return sign ? -v : v;
}

static double bf16_value(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* O_F64 holds exact values given as doubles (e.g. dequantised E4M3 queries:
 * a 4-bit significand times an fp32 scale fits a double). */
static double load_elem(const void *base, int dtype, int64_t i)
{
    if (dtype == O_F64)
        return ((const double *)base)[i];
    if (dtype == O_F32)
        return (double)((const float *)base)[i];
    if (dtype == O_BF16)
        return bf16_value(((const uint16_t *)base)[i]);
    return ds4o_e4m3_decode(((const uint8_t *)base)[i]);
}

typedef struct {
    const void *q;
    int q_dtype;
    const void *k;
    int k_dtype;
    const float *k_scale;
    const float *w;
    int B, T, S, H, D;
    int64_t offset;
} problem;

/* Key row s of batch b, decoded to exact doubles (times its scale for fp8). */
static void key_row(const problem *p, int b, int64_t s, double *out)
{
    int64_t base = ((int64_t)b * p->S + s) * p->D;
    double sc = 1.0;
    if (p->k_dtype == O_FP8)
        sc = (double)p->k_scale[(int64_t)b * p->S + s];
    for (int d = 0; d < p->D; d++)
        out[d] = load_elem(p->k, p->k_dtype, base + d) * sc;
}

/* Query token (b, t): its H x D query block and H head weights, as doubles. */
static void query_block(const problem *p, int b, int t, double *qd, double *wd)
{
    int64_t base = ((int64_t)b * p->T + t) * p->H;
    for (int h = 0; h < p->H; h++) {
        wd[h] = (double)p->w[base + h];
        for (int d = 0; d < p->D; d++)
            qd[(int64_t)h * p->D + d] = load_elem(p->q, p->q_dtype, (base + h) * p->D + d);
    }
}

/* score(t, s) = sum_h w[t,h] * max(0, q[t,h,:] . k[s,:]) */
static double score_one(const problem *p, const double *qd, const double *wd, const double *kd)
{
    double score = 0.0;
    for (int h = 0; h < p->H; h++) {
        double dot = 0.0;
        const double *qh = qd + (int64_t)h * p->D;
        for (int d = 0; d < p->D; d++)
            dot += qh[d] * kd[d];
        score += wd[h] * (dot > 0.0 ? dot : 0.0);
    }
    return score;
}

typedef struct {
    double score;
    int64_t s;
} entry;

/* (score descending, index ascending). */
static int by_score_then_index(const void *a, const void *b)
{
    const entry *x = (const entry *)a, *y = (const entry *)b;
    if (x->score > y->score) return -1;
    if (x->score < y->score) return 1;
    return (x->s > y->s) - (x->s < y->s);
}

static int by_index(const void *a, const void *b)
{
    const entry *x = (const entry *)a, *y = (const entry *)b;
    return (x->s > y->s) - (x->s < y->s);
}

static int set_threads(int nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
    return omp_get_max_threads();
#else
    (void)nthreads;
    return 1;
#endif
}

#define KEY_BLOCK 2048

/*
 * Top-k for a list of rows. rows[i] is a flat row id b*T + t.
 * Outputs per row i: idx[i*topk ..] ascending, -1 padded; val[i*topk ..] the
 * fp64 scores of those indices (NaN for padding); kth[i] the score of the
 * last selected key in (score desc, index asc) order; rms[i] the root mean
 * square of all visible scores of the row.
 * Returns the number of threads used, or -1 on a bad argument.
 */
int ds4o_select(const void *q, int q_dtype, const void *k, int k_dtype, const float *k_scale,
                const float *w, int B, int T, int S, int H, int D, int64_t offset, int topk,
                const int64_t *rows, int nrows, int32_t *idx, double *val, double *kth,
                double *rms, int nthreads)
{
    problem p = {q, q_dtype, k, k_dtype, k_scale, w, B, T, S, H, D, offset};
    if (B < 1 || T < 1 || S < 1 || H < 1 || D < 1 || topk < 1 || offset < 0 || offset + T > S)
        return -1;
    int used = set_threads(nthreads);

    entry **lists = (entry **)calloc((size_t)nrows, sizeof(entry *));
    int64_t *len = (int64_t *)calloc((size_t)nrows, sizeof(int64_t));
    int64_t *first_item = (int64_t *)calloc((size_t)nrows + 1, sizeof(int64_t));
    for (int i = 0; i < nrows; i++) {
        int t = (int)(rows[i] % T);
        len[i] = offset + t + 1;
        lists[i] = (entry *)malloc((size_t)len[i] * sizeof(entry));
        first_item[i + 1] = first_item[i] + (len[i] + KEY_BLOCK - 1) / KEY_BLOCK;
    }
    int64_t nitems = first_item[nrows];

    /* Scores: one work item per (row, block of keys). */
#pragma omp parallel
    {
        double *qd = (double *)malloc((size_t)H * D * sizeof(double));
        double *wd = (double *)malloc((size_t)H * sizeof(double));
        double *kd = (double *)malloc((size_t)D * sizeof(double));
        int cur_row = -1;
#pragma omp for schedule(dynamic, 1)
        for (int64_t it = 0; it < nitems; it++) {
            int i = 0;
            int lo = 0, hi = nrows - 1;
            while (lo < hi) { /* row whose item range holds it */
                int mid = (lo + hi + 1) / 2;
                if (first_item[mid] <= it) lo = mid; else hi = mid - 1;
            }
            i = lo;
            int b = (int)(rows[i] / T), t = (int)(rows[i] % T);
            if (cur_row != i) {
                query_block(&p, b, t, qd, wd);
                cur_row = i;
            }
            int64_t s0 = (it - first_item[i]) * KEY_BLOCK;
            int64_t s1 = s0 + KEY_BLOCK < len[i] ? s0 + KEY_BLOCK : len[i];
            for (int64_t s = s0; s < s1; s++) {
                key_row(&p, b, s, kd);
                lists[i][s].score = score_one(&p, qd, wd, kd);
                lists[i][s].s = s;
            }
        }
        free(qd);
        free(wd);
        free(kd);
    }

    /* Selection: order, take the first min(k, L), emit ascending. */
#pragma omp parallel for schedule(dynamic, 1)
    for (int i = 0; i < nrows; i++) {
        entry *e = lists[i];
        int64_t L = len[i];
        double ss = 0.0;
        for (int64_t s = 0; s < L; s++)
            ss += e[s].score * e[s].score;
        rms[i] = sqrt(ss / (double)L);
        qsort(e, (size_t)L, sizeof(entry), by_score_then_index);
        int64_t m = L < topk ? L : topk;
        kth[i] = e[m - 1].score;
        qsort(e, (size_t)m, sizeof(entry), by_index);
        for (int64_t j = 0; j < topk; j++) {
            idx[(int64_t)i * topk + j] = j < m ? (int32_t)e[j].s : -1;
            val[(int64_t)i * topk + j] = j < m ? e[j].score : NAN;
        }
        free(lists[i]);
    }
    free(lists);
    free(len);
    free(first_item);
    return used;
}

/*
 * Scores at arbitrary (row, key) pairs: out[i] = score(rows[i], keys[i]), or
 * NaN when the key is not visible to the row (key > offset + t).
 */
int ds4o_score_pairs(const void *q, int q_dtype, const void *k, int k_dtype, const float *k_scale,
                     const float *w, int B, int T, int S, int H, int D, int64_t offset,
                     const int64_t *rows, const int64_t *keys, int64_t n, double *out,
                     int nthreads)
{
    problem p = {q, q_dtype, k, k_dtype, k_scale, w, B, T, S, H, D, offset};
    if (B < 1 || T < 1 || S < 1 || H < 1 || D < 1 || offset < 0 || offset + T > S)
        return -1;
    int used = set_threads(nthreads);
#pragma omp parallel
    {
        double *qd = (double *)malloc((size_t)H * D * sizeof(double));
        double *wd = (double *)malloc((size_t)H * sizeof(double));
        double *kd = (double *)malloc((size_t)D * sizeof(double));
#pragma omp for schedule(dynamic, 64)
        for (int64_t i = 0; i < n; i++) {
            int b = (int)(rows[i] / T), t = (int)(rows[i] % T);
            if (keys[i] < 0 || keys[i] > offset + t) {
                out[i] = NAN;
                continue;
            }
            query_block(&p, b, t, qd, wd);
            key_row(&p, b, keys[i], kd);
            out[i] = score_one(&p, qd, wd, kd);
        }
        free(qd);
        free(wd);
        free(kd);
    }
    return used;
}
