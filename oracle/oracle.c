/*
 * oracle.c -- plain, slow, fp64 CPU implementation of differential attention.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg load this library. It shares no code,
 * header, helper or constant with the HIP path and is never a fallback for it.
 *
 * Every function follows the definitions on the source pages:
 *   [L]  lesson "Differential Attention (V2)" (AI Engineering from Scratch,
 *        phase 10 lesson 16), section "Concept": the softmax weights
 *        w_i = exp(q.k_i/sqrt(d)) / sum_j exp(q.k_j/sqrt(d)); the two maps
 *        A1 = softmax(Q1 K1^T/sqrt(d)), A2 = softmax(Q2 K2^T/sqrt(d)); the
 *        output (A1 - lambda A2) V; and lambda = exp(lq1.lk1) - exp(lq2.lk2)
 *        + lambda_init, a per-head scalar.
 *   [L1] same lesson, "Build it", step 1: softmax computed by subtracting the
 *        row maximum, exponentiating, summing and dividing.
 *   [L3] same lesson, "Build it", step 3: the combined weight a1 - lambda a2
 *        per key, then the weighted sum of value rows.
 *   [VV] same lesson, "V1 vs V2": V1 applies a per-head RMSNorm after the
 *        difference; V2 drops it and keeps the KV heads of GQA while doubling
 *        the query heads.
 *   [HF] the community post on the DIFF Transformer: GroupNorm for each head
 *        (the mean-subtracting variant of the per-head norm).
 *   [AV] lesson "Attention Variants" (phase 7 lesson 15), "Build it", step 1:
 *        the causal mask admits key j for query i iff j <= i; step 2 and the
 *        sliding-window figure of its "Concept" section: a causal window of W
 *        admits key j iff i - W + 1 <= j <= i (W keys, the query's own
 *        included; W >= N is the full causal mask).
 *   [SK] the integrator skill page of the same lesson: the default depth
 *        schedule lambda_init = 0.8 - 0.6 exp(-0.3 (depth - 1)).
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *   - sqrt(d) uses d = d_qk, the dimension of the dot product (a caller may
 *     pass another scale);
 *   - GQA: output head h reads KV head h / (H / H_kv);
 *   - V1 norm: RMS over the d_v channels of one (token, head),
 *     y = o / sqrt(mean(o^2) + eps) * gamma[h] * (1 - lambda_init);
 *   - decode: the new token's key/value are already in the cache, the query
 *     attends to all ctx_len tokens; token t lives in physical page
 *     page_table[b][t / page], slot t % page.
 *
 * Inputs are fp32 arrays (bf16 inputs are widened exactly by the caller);
 * all arithmetic is fp64 and every sum runs in index order (built without
 * contraction into fused multiply-adds and without reassociation, so the
 * compiler's vectorisation across independent sums changes no result).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* [SK] default lambda_init schedule; depth is the 1-based layer index. */
double oracle_lambda_init(int depth)
{
    return 0.8 - 0.6 * exp(-0.3 * (double)(depth - 1));
}

/* [L] lambda_h = exp(lq1_h . lk1_h) - exp(lq2_h . lk2_h) + lambda_init(depth).
 * Vectors are [H, d_l] row-major. */
void oracle_lambda(const float *lq1, const float *lk1, const float *lq2,
                   const float *lk2, int H, int d_l, int depth, double *out)
{
    double init = oracle_lambda_init(depth);
    for (int h = 0; h < H; ++h) {
        double d1 = 0.0, d2 = 0.0;
        for (int k = 0; k < d_l; ++k) {
            d1 += (double)lq1[(int64_t)h * d_l + k] * (double)lk1[(int64_t)h * d_l + k];
            d2 += (double)lq2[(int64_t)h * d_l + k] * (double)lk2[(int64_t)h * d_l + k];
        }
        out[h] = exp(d1) - exp(d2) + init;
    }
}

/* [L1] softmax of s[0..n) in place: subtract the maximum, exponentiate,
 * sum, divide. */
static void softmax_inplace(double *s, int64_t n)
{
    double m = s[0];
    for (int64_t j = 1; j < n; ++j)
        if (s[j] > m) m = s[j];
    double sum = 0.0;
    for (int64_t j = 0; j < n; ++j) {
        s[j] = exp(s[j] - m);
        sum += s[j];
    }
    for (int64_t j = 0; j < n; ++j)
        s[j] /= sum;
}

static double dot(const float *a, const float *b, int d)
{
    double acc = 0.0;
    for (int k = 0; k < d; ++k)
        acc += (double)a[k] * (double)b[k];
    return acc;
}

/* q . b[0], ..., q . b[3]: four dot products formed side by side, each
 * summed in index order exactly as dot() sums it (the four sums are
 * independent, so evaluating them together changes no result, only the
 * speed). */
static void dot4(const float *q, const float *const *b, int d, double out[4])
{
    double s0 = 0.0, s1 = 0.0, s2 = 0.0, s3 = 0.0;
    for (int k = 0; k < d; ++k) {
        const double x = (double)q[k];
        s0 += x * (double)b[0][k];
        s1 += x * (double)b[1][k];
        s2 += x * (double)b[2][k];
        s3 += x * (double)b[3][k];
    }
    out[0] = s0;
    out[1] = s1;
    out[2] = s2;
    out[3] = s3;
}

/* One output row. kp1/kp2/vp hold the n visible keys/values in key order.
 * Scratch s1, s2 hold n doubles each. Writes y[0..d_v). */
static void diff_row(const float *q1, const float *q2,
                     const float *const *kp1, const float *const *kp2,
                     const float *const *vp, int64_t n, int d_qk, int d_v,
                     double lambda, double scale, int norm, const float *gamma,
                     double eps, double lambda_init, double *s1, double *s2,
                     double *y)
{
    if (n <= 0) { /* no visible key: defined as a zero row */
        for (int c = 0; c < d_v; ++c) y[c] = 0.0;
        return;
    }
    /* [L] scores of both branches (four keys at a time, then the rest) */
    int64_t j0 = 0;
    for (; j0 + 4 <= n; j0 += 4) {
        double d1[4], d2[4];
        dot4(q1, kp1 + j0, d_qk, d1);
        dot4(q2, kp2 + j0, d_qk, d2);
        for (int t = 0; t < 4; ++t) {
            s1[j0 + t] = d1[t] * scale;
            s2[j0 + t] = d2[t] * scale;
        }
    }
    for (int64_t j = j0; j < n; ++j) {
        s1[j] = dot(q1, kp1[j], d_qk) * scale;
        s2[j] = dot(q2, kp2[j], d_qk) * scale;
    }
    /* [L1] the two maps */
    softmax_inplace(s1, n);
    softmax_inplace(s2, n);
    /* [L3] combined weight per key, then the weighted sum of values */
    for (int c = 0; c < d_v; ++c) y[c] = 0.0;
    for (int64_t j = 0; j < n; ++j) {
        double w = s1[j] - lambda * s2[j];
        const float *vr = vp[j];
        for (int c = 0; c < d_v; ++c)
            y[c] += w * (double)vr[c];
    }
    /* [VV] V1: per-head norm after the difference, scaled by (1 - lambda_init):
     * norm 1 RMSNorm; norm 2 GroupNorm with one group per head ([HF]): the
     * channel mean is subtracted first and the variance replaces the mean square */
    if (norm) {
        double mu = 0.0;
        if (norm == 2) {
            for (int c = 0; c < d_v; ++c) mu += y[c];
            mu /= (double)d_v;
            for (int c = 0; c < d_v; ++c) y[c] -= mu;
        }
        double ms = 0.0;
        for (int c = 0; c < d_v; ++c) ms += y[c] * y[c];
        ms /= (double)d_v;
        double r = 1.0 / sqrt(ms + eps);
        for (int c = 0; c < d_v; ++c)
            y[c] = y[c] * r * (double)gamma[c] * (1.0 - lambda_init);
    }
}

/*
 * Prefill. Layouts (row-major, contiguous):
 *   q1, q2 [B, H, N, d_qk]; k1, k2 [B, H_kv, N, d_qk]; v [B, H_kv, N, d_v];
 *   lambda [H]; gamma [H, d_v] (used when norm != 0).
 * window: 0 for none, else the causal sliding window W (needs causal).
 * rows: flat row ids r = (b * H + h) * N + i to compute (NULL: all B*H*N rows,
 * in that order); out [nrows, d_v] fp64.
 * Returns 0, or -1 on an invalid argument.
 */
int oracle_prefill(const float *q1, const float *q2, const float *k1,
                   const float *k2, const float *v, int B, int H, int H_kv,
                   int N, int d_qk, int d_v, const double *lambda, int depth,
                   int causal, int window, double scale, int norm, const float *gamma,
                   double eps, const int64_t *rows, int64_t nrows, double *out)
{
    if (B < 0 || H <= 0 || H_kv <= 0 || N < 0 || d_qk <= 0 || d_v <= 0) return -1;
    if (H % H_kv != 0) return -1;
    if (window < 0 || (window > 0 && !causal)) return -1;
    if (norm && !gamma) return -1;
    int64_t total = (int64_t)B * H * N;
    if (!rows) nrows = total;
    const int group = H / H_kv;
    const double init = oracle_lambda_init(depth);
    int bad = 0;

#pragma omp parallel
    {
        double *s1 = (double *)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
        double *s2 = (double *)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
        const float **kp1 = (const float **)malloc(sizeof(void *) * (size_t)(N > 0 ? N : 1));
        const float **kp2 = (const float **)malloc(sizeof(void *) * (size_t)(N > 0 ? N : 1));
        const float **vp = (const float **)malloc(sizeof(void *) * (size_t)(N > 0 ? N : 1));
#pragma omp for schedule(dynamic, 1)
        for (int64_t t = 0; t < nrows; ++t) {
            int64_t r = rows ? rows[t] : t;
            if (r < 0 || r >= total) { bad = 1; continue; }
            int64_t i = r % N;
            int64_t bh = r / N;
            int h = (int)(bh % H);
            int b = (int)(bh / H);
            int g = h / group;
            int64_t lo = 0, hi = N;                /* visible keys [lo, hi) */
            if (causal) hi = i + 1;                /* [AV] j <= i */
            if (window > 0 && i - window + 1 > 0) lo = i - window + 1; /* [AV] window */
            int64_t n = hi - lo;
            int64_t kvbase = ((int64_t)b * H_kv + g) * N;
            for (int64_t j = 0; j < n; ++j) {
                kp1[j] = k1 + (kvbase + lo + j) * d_qk;
                kp2[j] = k2 + (kvbase + lo + j) * d_qk;
                vp[j] = v + (kvbase + lo + j) * d_v;
            }
            diff_row(q1 + r * d_qk, q2 + r * d_qk, kp1, kp2, vp, n, d_qk, d_v,
                     lambda[h], scale, norm, norm ? gamma + (int64_t)h * d_v : NULL,
                     eps, init, s1, s2, out + t * d_v);
        }
        free(s1); free(s2); free(kp1); free(kp2); free(vp);
    }
    return bad ? -1 : 0;
}

/*
 * Paged decode: one query token per sequence.
 *   q1, q2 [B, H, d_qk]; k1c, k2c [P, H_kv, page, d_qk]; vc [P, H_kv, page, d_v];
 *   page_table [B, max_pages]; ctx_len [B]; lambda [H]; gamma [H, d_v].
 * window: 0 for none, else the query (token L-1) sees tokens L-W .. L-1
 *   ([AV] causal window, read for the last row of a sequence).
 * out [B, H, d_v] fp64. Returns 0, or -1 on an invalid argument or page id.
 */
int oracle_decode(const float *q1, const float *q2, const float *k1c,
                  const float *k2c, const float *vc, int B, int H, int H_kv,
                  int d_qk, int d_v, int page, int max_pages, int num_pages,
                  const int32_t *page_table, const int32_t *ctx_len,
                  const double *lambda, int depth, int window, double scale, int norm,
                  const float *gamma, double eps, double *out)
{
    if (B < 0 || H <= 0 || H_kv <= 0 || d_qk <= 0 || d_v <= 0 || page <= 0) return -1;
    if (window < 0) return -1;
    if (H % H_kv != 0) return -1;
    if (norm < 0 || norm > 2 || (norm && !gamma)) return -1;
    const int group = H / H_kv;
    const double init = oracle_lambda_init(depth);
    int64_t maxlen = (int64_t)max_pages * page;
    int bad = 0;

#pragma omp parallel
    {
        double *s1 = (double *)malloc(sizeof(double) * (size_t)(maxlen > 0 ? maxlen : 1));
        double *s2 = (double *)malloc(sizeof(double) * (size_t)(maxlen > 0 ? maxlen : 1));
        const float **kp1 = (const float **)malloc(sizeof(void *) * (size_t)(maxlen > 0 ? maxlen : 1));
        const float **kp2 = (const float **)malloc(sizeof(void *) * (size_t)(maxlen > 0 ? maxlen : 1));
        const float **vp = (const float **)malloc(sizeof(void *) * (size_t)(maxlen > 0 ? maxlen : 1));
#pragma omp for schedule(dynamic, 1)
        for (int64_t t = 0; t < (int64_t)B * H; ++t) {
            int b = (int)(t / H), h = (int)(t % H), g = h / group;
            int64_t L = ctx_len[b];
            if (L < 0 || L > maxlen) { bad = 1; continue; }
            int64_t lo = (window > 0 && L > window) ? L - window : 0; /* visible tokens [lo, L) */
            int ok = 1;
            for (int64_t j = lo; j < L; ++j) {
                int32_t phys = page_table[(int64_t)b * max_pages + j / page];
                if (phys < 0 || phys >= num_pages) { ok = 0; break; }
                int64_t base = (((int64_t)phys * H_kv + g) * page + j % page);
                kp1[j - lo] = k1c + base * d_qk;
                kp2[j - lo] = k2c + base * d_qk;
                vp[j - lo] = vc + base * d_v;
            }
            if (!ok) { bad = 1; continue; }
            diff_row(q1 + t * d_qk, q2 + t * d_qk, kp1, kp2, vp, L - lo, d_qk, d_v,
                     lambda[h], scale, norm, norm ? gamma + (int64_t)h * d_v : NULL,
                     eps, init, s1, s2, out + t * d_v);
        }
        free(s1); free(s2); free(kp1); free(kp2); free(vp);
    }
    return bad ? -1 : 0;
}

/* Threads the OpenMP runtime will use (for reporting). */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
