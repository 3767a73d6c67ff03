/*
 * CPU oracle for sparse attention over the indexer's selected positions.
 *
 * TEST INFRASTRUCTURE. Like ds4idx_oracle.c, this is the plain reference the
 * HIP kernel is checked against; only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may build, load or call it. It shares nothing
 * with the HIP library.
 *
 * What it computes. Sparse attention attends each query token only to a
 * selected subset of positions (first page, "DeepSeek V4 Flash 추론을 1.6초로
 * 줄인 ds4 최적화", glossary entry on sparse attention), the subset the
 * Lightning Indexer picks. The MI300X write-up ("DeepSeek V4 Flash는 단일 AMD
 * MI300X에서 실행됩니다") names the cache format fp8_ds_mla (deployment
 * checklist, hybrid KV strategy) and tiles the sparse prefill 64 heads at a
 * time (production tuning table, BLOCK_H=64). The plainest reading is
 * attention over a shared latent cache (MLA): every cache row c[s] (d_qk
 * values) serves as the key of all heads, its first d_v values as the value:
 *
 *   for each stream b, token t, head h, over the valid entries j of idx[b,t]
 *   (0 <= idx < S; -1 padding and anything else out of range is skipped):
 *     z_j = softmax_scale * sum_d q[b,t,h,d] * c[b, idx_j, d]
 *     out[b,t,h,:] = sum_j exp(z_j - m) c[b, idx_j, 0:d_v] / sum_j exp(z_j - m),  m = max_j z_j
 *     lse[b,t,h]   = m + log(sum_j exp(z_j - m))
 *   A token with no valid entry gets out = 0 and lse = -inf.
 *
 * Arithmetic in double: products of bf16 values are exact, dot products are
 * summed in index order, exp/log from libm.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double bf16d(uint16_t b)
{
    const uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/*
 * q [B,T,H,d_qk] bf16 bits, c [B,S,d_qk] bf16 bits, idx [B,T,k] int32.
 * For the flat (b*T + t) rows listed in rows[0..nrows): out [nrows,H,d_v]
 * and lse [nrows,H], doubles. Returns the threads used, or -1 on a bad
 * argument.
 */
int ds4o_sparse_attention(const uint16_t *q, const uint16_t *c, const int32_t *idx, int B, int T,
                          int S, int H, int k, int d_qk, int d_v, double softmax_scale,
                          const int64_t *rows, int nrows, double *out, double *lse, int nthreads)
{
    if (B < 1 || T < 1 || S < 1 || H < 1 || k < 1 || d_qk < 1 || d_v < 1 || d_v > d_qk)
        return -1;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
    const int used = omp_get_max_threads();
#else
    (void)nthreads;
    const int used = 1;
#endif
#pragma omp parallel
    {
        double *z = (double *)malloc((size_t)k * sizeof(double));
        int64_t *sel = (int64_t *)malloc((size_t)k * sizeof(int64_t));
#pragma omp for schedule(dynamic, 1) collapse(2)
        for (int i = 0; i < nrows; i++) {
            for (int h = 0; h < H; h++) {
                const int64_t r = rows[i];
                const int64_t b = r / T;
                int n = 0;
                for (int j = 0; j < k; j++) {
                    const int32_t s = idx[r * k + j];
                    if (s >= 0 && s < S)
                        sel[n++] = s;
                }
                double *o = out + ((int64_t)i * H + h) * d_v;
                for (int d = 0; d < d_v; d++)
                    o[d] = 0.0;
                if (n == 0) {
                    lse[(int64_t)i * H + h] = -INFINITY;
                    continue;
                }
                const uint16_t *qh = q + ((r * H) + h) * (int64_t)d_qk;
                double m = -INFINITY;
                for (int j = 0; j < n; j++) {
                    const uint16_t *cr = c + (b * S + sel[j]) * (int64_t)d_qk;
                    double dot = 0.0;
                    for (int d = 0; d < d_qk; d++)
                        dot += bf16d(qh[d]) * bf16d(cr[d]);
                    z[j] = softmax_scale * dot;
                    if (z[j] > m)
                        m = z[j];
                }
                double l = 0.0;
                for (int j = 0; j < n; j++) {
                    const double p = exp(z[j] - m);
                    l += p;
                    const uint16_t *cr = c + (b * S + sel[j]) * (int64_t)d_qk;
                    for (int d = 0; d < d_v; d++)
                        o[d] += p * bf16d(cr[d]);
                }
                for (int d = 0; d < d_v; d++)
                    o[d] /= l;
                lse[(int64_t)i * H + h] = m + log(l);
            }
        }
        free(z);
        free(sel);
    }
    return used;
}
