/*
 * gdla_oracle.c -- CPU oracle for the attention core of Grouped Differential
 * Latent Attention (GDLA).  TEST INFRASTRUCTURE ONLY: the tests, the smoke
 * check and the CPU baseline of the benchmark call it; the product library
 * never links or loads it, and it shares no code with the HIP kernels.
 *
 * What it computes is the plain definition, written out with no tiling, no
 * online softmax and no fusion.  Sources (web pages on the Motif 3 technical
 * report):
 *   - aitrends.kr "314B MoE 언어 모델 Motif 3의 구조와 학습 시스템",
 *     GDLA paragraph: the signal and noise paths share one KV head, each runs
 *     its own attention, then D_t = H_S,t - lambda_t (.) Repeat_g(H_N,t), then
 *     a query-based element-wise gate, then the output projection.
 *   - same page, grouped-differential paragraph: g = 4, n_N = n_H/(g+1),
 *     n_S = g*n_N; each signal head pairs with the noise head of its group.
 *   - same page, first GDLA paragraph: each noise-head output is repeated to
 *     its four corresponding signal heads; lambda_t = sigmoid(x_t W^lambda)
 *     lies in (0,1).
 *   - same page, context-parallel paragraph, and idailynews (page 5): the
 *     sliding-window layers see a 128-token window; full layers see the whole
 *     causal prefix.
 *   - metalmedia (page 2), Table 1: 80 query / 16 KV heads, 64 signal / 16
 *     noise, query-key head dim 192, value head dim 128.
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *   - the window covers keys t-W+1 .. t inclusive (W = 0 means full causal);
 *   - Repeat_g is an interleave: noise head j feeds signal heads g*j..g*j+g-1,
 *     and that whole group reads KV head j;
 *   - lambda is one scalar per (token, signal head), used as given;
 *   - no normalisation between the subtraction and the gate;
 *   - the softmax scale is an argument (callers pass 1/sqrt(d_qk)).
 *
 * Arithmetic: inputs are fp32 arrays (bf16 inputs widen to fp32 exactly);
 * every product, sum and exponential is carried in fp64, and the result is
 * returned in fp64 with no rounding.  The softmax takes two passes over the
 * scores: first the scores and their maximum, then exp(z - max), the sum and
 * the weighted sum of values.
 *
 * Parallelism: independent output rows are spread over OpenMP threads; this
 * changes no arithmetic, since every row is computed by one thread in the
 * same sequential order.
 *
 * Compile-time switch ORACLE_MUTANT (tests only): when defined to k > 0, a
 * deliberate mistake number k is planted, so that the tests can show that
 * their pins catch it.  The normal build leaves it undefined.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>

#ifndef ORACLE_MUTANT
#define ORACLE_MUTANT 0
#endif

enum { ORACLE_OK = 0, ORACLE_BAD_ARG = 1, ORACLE_NO_MEMORY = 2 };

/*
 * Softmax attention of one query vector q[d_qk] over the keys s_lo..s_hi-1
 * (inclusive of s_lo, exclusive of s_hi) of one KV head:
 *   z_s = scale * sum_d q[d] k_s[d]
 *   out = sum_s exp(z_s - max z) v_s / sum_s exp(z_s - max z)
 * Key row s lives at k + s*k_stride, value row s at v + s*v_stride.
 * z is caller scratch of at least s_hi - s_lo doubles.
 */
static void attend_one(const float *q, const float *k, long k_stride,
                       const float *v, long v_stride, long s_lo, long s_hi,
                       int d_qk, int d_v, double scale, double *z, double *out)
{
    double zmax = -INFINITY;
    for (long s = s_lo; s < s_hi; ++s) {
        const float *ks = k + s * k_stride;
        double dot = 0.0;
#if ORACLE_MUTANT == 5
        for (int d = 0; d + 64 < d_qk; ++d)      /* planted: drops the 64-dim rotary tail */
#else
        for (int d = 0; d < d_qk; ++d)
#endif
            dot += (double)q[d] * (double)ks[d];
#if ORACLE_MUTANT == 6
        z[s - s_lo] = dot;                       /* planted: forgets the scale */
        (void)scale;
#else
        z[s - s_lo] = scale * dot;
#endif
        if (z[s - s_lo] > zmax)
            zmax = z[s - s_lo];
    }
    double denom = 0.0;
    for (int c = 0; c < d_v; ++c)
        out[c] = 0.0;
    for (long s = s_lo; s < s_hi; ++s) {
        double e = exp(z[s - s_lo] - zmax);
        denom += e;
        const float *vs = v + s * v_stride;
        for (int c = 0; c < d_v; ++c)
            out[c] += e * (double)vs[c];
    }
    for (int c = 0; c < d_v; ++c)
        out[c] /= denom;
}

/* First visible key for a query at position t: t-W+1 with a window, else 0. */
static long first_visible(long t, int window)
{
#if ORACLE_MUTANT == 3
    long lo = window > 0 ? t - window : 0;       /* planted: window one key too wide */
#else
    long lo = window > 0 ? t - window + 1 : 0;
#endif
    return lo > 0 ? lo : 0;
}

/*
 * One group (KV head j, its noise head and its `group` signal heads) for one
 * query position: H_N from the noise query, H_S from each signal query, then
 *   D[h][c] = H_S[h][c] - lambda[h] * H_N[c]   (Repeat_g as interleave:
 *                                               signal head g*j+i uses noise head j)
 *   O[h][c] = gate[h][c] * D[h][c]
 * qs points at the group's first signal query, qn_row at the row's first noise
 * query ([n_kv][d_qk]), lam/gate/out at the group's first signal head.
 */
static void group_row(const float *qs, const float *qn_row, int j, int n_kv,
                      const float *k, long k_stride, const float *v, long v_stride,
                      long s_lo, long s_hi, int group, int d_qk, int d_v, double scale,
                      const float *lam, const float *gate, double *z,
                      double *h_noise, double *h_sig, double *out)
{
    attend_one(qn_row + (long)j * d_qk, k, k_stride, v, v_stride, s_lo, s_hi, d_qk, d_v,
               scale, z, h_noise);
    for (int i = 0; i < group; ++i) {
#if ORACLE_MUTANT == 1
        /* planted: Repeat_g as a tile -- signal head h pairs with noise head h mod n_kv */
        attend_one(qn_row + (long)((j * group + i) % n_kv) * d_qk, k, k_stride, v, v_stride,
                   s_lo, s_hi, d_qk, d_v, scale, z, h_noise);
#else
        (void)n_kv;
#endif
        attend_one(qs + (long)i * d_qk, k, k_stride, v, v_stride, s_lo, s_hi,
                   d_qk, d_v, scale, z, h_sig);
        for (int c = 0; c < d_v; ++c) {
#if ORACLE_MUTANT == 2
            double d = h_sig[c] + (double)lam[i] * h_noise[c];   /* planted: wrong sign */
#else
            double d = h_sig[c] - (double)lam[i] * h_noise[c];
#endif
#if ORACLE_MUTANT == 4
            out[(long)i * d_v + c] = d;                          /* planted: gate not applied */
            (void)gate;
#else
            out[(long)i * d_v + c] = (double)gate[(long)i * d_v + c] * d;
#endif
        }
    }
}

static int dims_ok(int n_kv, int group, int d_qk, int d_v)
{
    return n_kv >= 1 && group >= 1 && d_qk >= 1 && d_v >= 1;
}

/*
 * Prefill for an arbitrary list of query positions.
 *   k        [B][T][n_kv][d_qk]   v [B][T][n_kv][d_v]
 *   row_b, row_t [n_rows]         which (sequence, position) each row is
 *   q_signal [n_rows][n_kv*group][d_qk]
 *   q_noise  [n_rows][n_kv][d_qk]
 *   lam      [n_rows][n_kv*group]
 *   gate     [n_rows][n_kv*group][d_v]
 *   out      [n_rows][n_kv*group][d_v]   (fp64)
 * window = 0: full causal (keys 0..t); window W >= 1: keys max(0,t-W+1)..t.
 * The full prefill is the special case n_rows = B*T with rows in (b, t)
 * order, where the per-row arrays are simply the full [B][T][...] tensors.
 */
int gdla_oracle_prefill_rows(const float *k, const float *v, int B, int T, int n_kv,
                             int group, int d_qk, int d_v, int window, double scale,
                             long n_rows, const int32_t *row_b, const int32_t *row_t,
                             const float *q_signal, const float *q_noise,
                             const float *lam, const float *gate, double *out)
{
    if (n_rows < 0 || B < 0 || T < 0 || window < 0 || !dims_ok(n_kv, group, d_qk, d_v))
        return ORACLE_BAD_ARG;
    if (n_rows == 0)
        return ORACLE_OK;
    if (!k || !v || !row_b || !row_t || !q_signal || !q_noise || !lam || !gate || !out)
        return ORACLE_BAD_ARG;
    for (long r = 0; r < n_rows; ++r)
        if (row_b[r] < 0 || row_b[r] >= B || row_t[r] < 0 || row_t[r] >= T)
            return ORACLE_BAD_ARG;

    const int n_sig = n_kv * group;
    const long k_stride = (long)n_kv * d_qk;     /* distance between key rows s, s+1 */
    const long v_stride = (long)n_kv * d_v;
    int failed = 0;

#pragma omp parallel
    {
        double *z = (double *)malloc(sizeof(double) * (size_t)T);
        double *hn = (double *)malloc(sizeof(double) * (size_t)d_v);
        double *hs = (double *)malloc(sizeof(double) * (size_t)d_v);
        if (!z || !hn || !hs) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (long w = 0; w < n_rows * n_kv; ++w) {
                const long r = w / n_kv;
                const int j = (int)(w % n_kv);
                const long b = row_b[r], t = row_t[r];
                const float *kb = k + ((long)b * T * n_kv + j) * d_qk;
#if ORACLE_MUTANT == 7
                const float *vb = v + ((long)b * T * n_kv + (j + 1) % n_kv) * d_v;  /* planted: V of the wrong KV head */
#else
                const float *vb = v + ((long)b * T * n_kv + j) * d_v;
#endif
                group_row(q_signal + (r * n_sig + (long)j * group) * d_qk,
                          q_noise + r * n_kv * d_qk, j, n_kv,
                          kb, k_stride, vb, v_stride, first_visible(t, window), t + 1,
                          group, d_qk, d_v, scale,
                          lam + r * n_sig + (long)j * group,
                          gate + (r * n_sig + (long)j * group) * d_v, z, hn, hs,
                          out + (r * n_sig + (long)j * group) * d_v);
            }
        }
        free(z);
        free(hn);
        free(hs);
    }
    return failed ? ORACLE_NO_MEMORY : ORACLE_OK;
}

/*
 * Decode: one new query per sequence, attending to that sequence's cache.
 *   q_signal [B][n_kv*group][d_qk]   q_noise [B][n_kv][d_qk]
 *   k_cache  [total][n_kv][d_qk]     v_cache [total][n_kv][d_v]
 *   cu_seqlens [B+1]: sequence b owns cache rows cu[b] .. cu[b+1]-1; its
 *   length L_b = cu[b+1]-cu[b] >= 1 already includes the new token, so the
 *   query sits at position L_b-1 and sees keys max(0, L_b-W) .. L_b-1.
 *   lam [B][n_kv*group]  gate, out [B][n_kv*group][d_v]
 */
int gdla_oracle_decode(const float *q_signal, const float *q_noise, const float *k_cache,
                       const float *v_cache, const int32_t *cu_seqlens, const float *lam,
                       const float *gate, int B, int n_kv, int group, int d_qk, int d_v,
                       int window, double scale, double *out)
{
    if (B < 0 || window < 0 || !dims_ok(n_kv, group, d_qk, d_v))
        return ORACLE_BAD_ARG;
    if (B == 0)
        return ORACLE_OK;
    if (!q_signal || !q_noise || !k_cache || !v_cache || !cu_seqlens || !lam || !gate || !out)
        return ORACLE_BAD_ARG;
    long max_len = 0;
    for (int b = 0; b < B; ++b) {
        long len = (long)cu_seqlens[b + 1] - cu_seqlens[b];
        if (cu_seqlens[b] < 0 || len < 1)
            return ORACLE_BAD_ARG;
        if (len > max_len)
            max_len = len;
    }

    const int n_sig = n_kv * group;
    const long k_stride = (long)n_kv * d_qk;
    const long v_stride = (long)n_kv * d_v;
    int failed = 0;

#pragma omp parallel
    {
        double *z = (double *)malloc(sizeof(double) * (size_t)max_len);
        double *hn = (double *)malloc(sizeof(double) * (size_t)d_v);
        double *hs = (double *)malloc(sizeof(double) * (size_t)d_v);
        if (!z || !hn || !hs) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (long w = 0; w < (long)B * n_kv; ++w) {
                const long b = w / n_kv;
                const int j = (int)(w % n_kv);
                const long len = (long)cu_seqlens[b + 1] - cu_seqlens[b];
                const long t = len - 1;
                const float *kb = k_cache + ((long)cu_seqlens[b] * n_kv + j) * d_qk;
                const float *vb = v_cache + ((long)cu_seqlens[b] * n_kv + j) * d_v;
                group_row(q_signal + (b * n_sig + (long)j * group) * d_qk,
                          q_noise + b * n_kv * d_qk, j, n_kv,
                          kb, k_stride, vb, v_stride, first_visible(t, window), t + 1,
                          group, d_qk, d_v, scale,
                          lam + b * n_sig + (long)j * group,
                          gate + (b * n_sig + (long)j * group) * d_v, z, hn, hs,
                          out + (b * n_sig + (long)j * group) * d_v);
            }
        }
        free(z);
        free(hn);
        free(hs);
    }
    return failed ? ORACLE_NO_MEMORY : ORACLE_OK;
}

/* Number of OpenMP threads a parallel region of this library would use. */
int gdla_oracle_num_threads(void)
{
    int n = 1;
#pragma omp parallel
    {
#pragma omp single
        n = omp_get_num_threads();
    }
    return n;
}
