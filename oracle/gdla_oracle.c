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

/*
 * Arithmetic type of the prefill and decode definitions.  The normal build
 * carries every product, sum and exponential in fp64.  Built with
 * -DORACLE_FP32, the same source carries them in fp32 (exp becomes expf):
 * the plain fp32 CPU reference whose speed is reported beside the GPU's.
 * The latent decode and the pre-attention step are always fp64.
 */
#ifdef ORACLE_FP32
typedef float real;
#define EXP expf
#else
typedef double real;
#define EXP exp
#endif

/* Largest query-key head dim the prefill and decode definitions accept. */
#define ORACLE_MAX_DQK 1024

enum { ORACLE_OK = 0, ORACLE_BAD_ARG = 1, ORACLE_NO_MEMORY = 2 };

/*
 * Scores of one query vector q[d_qk] against the keys s_lo..s_hi-1 of one KV
 * head:  z[s - s_lo] = scale * sum_d q[d] k_s[d].  Each dot product is summed
 * over d in ascending order; eight keys are taken at a time only so that
 * their (independent) sums overlap in the CPU's pipeline.
 */
static void scores(const real *q, const float *k, long k_stride, long s_lo, long s_hi,
                   int d_qk, real scale, real *z)
{
#if ORACLE_MUTANT == 5
    const int d_end = d_qk - 64;                 /* planted: drops the 64-dim rotary tail */
#else
    const int d_end = d_qk;
#endif
    long s = s_lo;
    for (; s + 8 <= s_hi; s += 8) {
        const float *ks = k + s * k_stride;
        real acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        for (int d = 0; d < d_end; ++d) {
#pragma GCC unroll 8
            for (int u = 0; u < 8; ++u)
                acc[u] += q[d] * (real)ks[u * k_stride + d];
        }
        for (int u = 0; u < 8; ++u)
            z[s + u - s_lo] = acc[u];
    }
    for (; s < s_hi; ++s) {
        const float *ks = k + s * k_stride;
        real dot = 0;
        for (int d = 0; d < d_end; ++d)
            dot += q[d] * (real)ks[d];
        z[s - s_lo] = dot;
    }
    for (long i = 0; i < s_hi - s_lo; ++i)
#if ORACLE_MUTANT == 6
        (void)scale;                             /* planted: forgets the scale */
#else
        z[i] = scale * z[i];
#endif
}

/*
 * Softmax attention of one query vector q[d_qk] over the keys s_lo..s_hi-1
 * (inclusive of s_lo, exclusive of s_hi) of one KV head:
 *   z_s = scale * sum_d q[d] k_s[d]
 *   out = sum_s exp(z_s - max z) v_s / sum_s exp(z_s - max z)
 * Key row s lives at k + s*k_stride, value row s at v + s*v_stride.
 * z is caller scratch of at least s_hi - s_lo values.
 */
static void attend_one(const float *qf, const float *k, long k_stride,
                       const float *v, long v_stride, long s_lo, long s_hi,
                       int d_qk, int d_v, real scale, real *z, real *out)
{
    real q[ORACLE_MAX_DQK];
    for (int d = 0; d < d_qk; ++d)
        q[d] = (real)qf[d];
    scores(q, k, k_stride, s_lo, s_hi, d_qk, scale, z);
    real zmax = -INFINITY;
    for (long s = s_lo; s < s_hi; ++s)
        if (z[s - s_lo] > zmax)
            zmax = z[s - s_lo];
    real denom = 0;
    for (int c = 0; c < d_v; ++c)
        out[c] = 0;
    for (long s = s_lo; s < s_hi; ++s) {
        const real e = EXP(z[s - s_lo] - zmax);
        denom += e;
        const float *vs = v + s * v_stride;
        for (int c = 0; c < d_v; ++c)
            out[c] += e * (real)vs[c];
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
                      long s_lo, long s_hi, int group, int d_qk, int d_v, real scale,
                      const float *lam, const float *gate, real *z,
                      real *h_noise, real *h_sig, double *out)
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
            const real d = h_sig[c] + (real)lam[i] * h_noise[c];  /* planted: wrong sign */
#else
            const real d = h_sig[c] - (real)lam[i] * h_noise[c];
#endif
#if ORACLE_MUTANT == 4
            out[(long)i * d_v + c] = d;                          /* planted: gate not applied */
            (void)gate;
#else
            out[(long)i * d_v + c] = (real)gate[(long)i * d_v + c] * d;
#endif
        }
    }
}

static int dims_ok(int n_kv, int group, int d_qk, int d_v)
{
    return n_kv >= 1 && group >= 1 && d_qk >= 1 && d_qk <= ORACLE_MAX_DQK && d_v >= 1;
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
        real *z = (real *)malloc(sizeof(real) * (size_t)T);
        real *hn = (real *)malloc(sizeof(real) * (size_t)d_v);
        real *hs = (real *)malloc(sizeof(real) * (size_t)d_v);
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
                          group, d_qk, d_v, (real)scale,
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
        real *z = (real *)malloc(sizeof(real) * (size_t)max_len);
        real *hn = (real *)malloc(sizeof(real) * (size_t)d_v);
        real *hs = (real *)malloc(sizeof(real) * (size_t)d_v);
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
                          group, d_qk, d_v, (real)scale,
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

/*
 * Decode over a latent (compressed) KV cache.  Each cache row holds the
 * normalised compressed KV c (d_c values) followed by the decoupled rotary key
 * k^R (d_r values), shared by every KV head.  KV head j's key and value rows
 * are the up-projections (aitrends.kr, GDLA paragraph: the compressed KV is
 * normalised once, expanded to the 16 KV heads, and the rotary key is shared
 * by all of them):
 *   K_j[s] = [ W_uk[j] c_s ; k^R_s ]   (d_qk = d_kc + d_r values)
 *   V_j[s] =   W_uv[j] c_s             (d_v values)
 * with W_uk [n_kv][d_kc][d_c], W_uv [n_kv][d_v][d_c].  Everything else is the
 * decode definition above.  Here the keys and values are formed explicitly, in
 * fp64, for the visible rows of each sequence, and the softmax runs over them.
 *   latent  [total][d_c + d_r]
 *   q_signal [B][n_kv*group][d_kc + d_r]   (content part first, then rotary)
 */
int gdla_oracle_decode_latent(const float *q_signal, const float *q_noise, const float *latent,
                              const float *w_uk, const float *w_uv, const int32_t *cu_seqlens,
                              const float *lam, const float *gate, int B, int n_kv, int group,
                              int d_c, int d_r, int d_kc, int d_v, int window, double scale,
                              double *out)
{
    if (B < 0 || window < 0 || d_c < 1 || d_r < 0 || d_kc < 1 || !dims_ok(n_kv, group, d_kc + d_r, d_v))
        return ORACLE_BAD_ARG;
    if (B == 0)
        return ORACLE_OK;
    if (!q_signal || !q_noise || !latent || !w_uk || !w_uv || !cu_seqlens || !lam || !gate || !out)
        return ORACLE_BAD_ARG;
    long max_len = 0;
    for (int b = 0; b < B; ++b) {
        long len = (long)cu_seqlens[b + 1] - cu_seqlens[b];
        if (cu_seqlens[b] < 0 || len < 1)
            return ORACLE_BAD_ARG;
        if (len > max_len)
            max_len = len;
    }
    const int d_qk = d_kc + d_r, n_sig = n_kv * group, row = d_c + d_r;
    int failed = 0;

#pragma omp parallel
    {
        double *kx = (double *)malloc(sizeof(double) * (size_t)max_len * (size_t)d_qk);
        double *vx = (double *)malloc(sizeof(double) * (size_t)max_len * (size_t)d_v);
        double *z = (double *)malloc(sizeof(double) * (size_t)max_len);
        double *hn = (double *)malloc(sizeof(double) * (size_t)d_v);
        double *hs = (double *)malloc(sizeof(double) * (size_t)d_v);
        if (!kx || !vx || !z || !hn || !hs) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (long w = 0; w < (long)B * n_kv; ++w) {
                const long b = w / n_kv;
                const int j = (int)(w % n_kv);
                const long len = (long)cu_seqlens[b + 1] - cu_seqlens[b];
                const long s_lo = first_visible(len - 1, window), n = len - s_lo;
                /* the visible keys and values of KV head j, expanded */
                for (long i = 0; i < n; ++i) {
                    const float *lr = latent + ((long)cu_seqlens[b] + s_lo + i) * row;
                    for (int d = 0; d < d_kc; ++d) {
                        double acc = 0.0;
                        for (int c = 0; c < d_c; ++c)
#if ORACLE_MUTANT == 9
                            /* planted: W_uk read as [d_c][d_kc] */
                            acc += (double)w_uk[(long)j * d_kc * d_c + (long)c * d_kc + d] * (double)lr[c];
#else
                            acc += (double)w_uk[((long)j * d_kc + d) * d_c + c] * (double)lr[c];
#endif
                        kx[i * d_qk + d] = acc;
                    }
                    for (int d = 0; d < d_r; ++d)
#if ORACLE_MUTANT == 8
                        kx[i * d_qk + d_kc + d] = 0.0;           /* planted: rotary key dropped */
#else
                        kx[i * d_qk + d_kc + d] = (double)lr[d_c + d];
#endif
                    for (int d = 0; d < d_v; ++d) {
#if ORACLE_MUTANT == 10
                        const float *wr = w_uk + ((long)j * d_v + d) * d_c;   /* planted: V from W_uk */
#else
                        const float *wr = w_uv + ((long)j * d_v + d) * d_c;
#endif
                        double acc = 0.0;
                        for (int c = 0; c < d_c; ++c)
                            acc += (double)wr[c] * (double)lr[c];
                        vx[i * d_v + d] = acc;
                    }
                }
                /* noise head j, then the group's signal heads (interleave) */
                for (int hh = -1; hh < group; ++hh) {
                    const float *q = hh < 0 ? q_noise + (b * n_kv + j) * (long)d_qk
                                            : q_signal + (b * n_sig + (long)j * group + hh) * d_qk;
                    double *h = hh < 0 ? hn : hs;
                    double zmax = -INFINITY;
                    for (long i = 0; i < n; ++i) {
                        double dot = 0.0;
                        for (int d = 0; d < d_qk; ++d)
                            dot += (double)q[d] * kx[i * d_qk + d];
                        z[i] = scale * dot;
                        if (z[i] > zmax)
                            zmax = z[i];
                    }
                    double denom = 0.0;
                    for (int c = 0; c < d_v; ++c)
                        h[c] = 0.0;
                    for (long i = 0; i < n; ++i) {
                        const double e = exp(z[i] - zmax);
                        denom += e;
                        for (int c = 0; c < d_v; ++c)
                            h[c] += e * vx[i * d_v + c];
                    }
                    for (int c = 0; c < d_v; ++c)
                        h[c] /= denom;
                    if (hh < 0)
                        continue;
                    const long o = (b * n_sig + (long)j * group + hh) * d_v;
                    const double l = (double)lam[b * n_sig + (long)j * group + hh];
                    for (int c = 0; c < d_v; ++c)
                        out[o + c] = (double)gate[o + c] * (hs[c] - l * hn[c]);
                }
            }
        }
        free(kx);
        free(vx);
        free(z);
        free(hn);
        free(hs);
    }
    return failed ? ORACLE_NO_MEMORY : ORACLE_OK;
}

/*
 * ---- The step ahead of the attention core (rotary embedding, lambda, gate).
 *
 * Sources: aitrends.kr (page above), GDLA paragraph: the query path expands
 * the compressed query into a content query and a rotary query; the KV path
 * produces a decoupled rotary key next to the compressed KV; lambda_t =
 * sigmoid(x_t W^lambda) from the input hidden state; a query-based
 * element-wise gate follows the subtraction.  Head-dimension paragraph: the
 * rotary component is 64 values of the 192, and the rotary key is shared by
 * every KV head.  metalmedia (page 2), Table 1: hidden dimension 4,096 and
 * output gating.
 *
 * Readings where the pages are silent (listed in the design notes):
 *   - the rotary part is the last 64 of a head's 192 values (content first);
 *   - the rotation is the original rotary position embedding: adjacent pairs
 *     (2i, 2i+1) turn counter-clockwise by pos * theta^(-2i/64), i = 0..31,
 *     with the base theta an argument (10000 in the original);
 *   - token t of every sequence sits at position pos0 + t;
 *   - lambda is one scalar per (token, signal head): sigmoid of the dot
 *     product of x_t with row h of W^lambda [n_sig, d_model];
 *   - the gate's projection is an ordinary matmul outside this step; the step
 *     applies its sigmoid to the given pre-activations.
 */
static void rope64(const float *x, double pos, double theta, double *out)
{
    for (int i = 0; i < 32; ++i) {
#if ORACLE_MUTANT == 13
        const double freq = pow(theta, -(double)i / 64.0);
#else
        const double freq = pow(theta, -2.0 * i / 64.0);
#endif
        const double a = pos * freq;
        const double c = cos(a);
#if ORACLE_MUTANT == 12
        const double s = -sin(a);
#else
        const double s = sin(a);
#endif
#if ORACLE_MUTANT == 11
        const int i0 = i, i1 = i + 32;
#else
        const int i0 = 2 * i, i1 = 2 * i + 1;
#endif
        out[i0] = (double)x[i0] * c - (double)x[i1] * s;
        out[i1] = (double)x[i0] * s + (double)x[i1] * c;
    }
}

static double sigmoid(double z)
{
#if ORACLE_MUTANT == 14
    return z;
#else
    return 1.0 / (1.0 + exp(-z));
#endif
}

/*
 * Rotated query heads (content part copied, rotary part rotated), the rotated
 * shared key as it lands in each KV head's rotary part, lambda and the gate.
 *   q_signal [B,T,n_sig,d_qk], q_noise [B,T,n_kv,d_qk], k_rope [B,T,64],
 *   x [B,T,d_model], w_lambda [n_sig,d_model], gate_pre [B,T,n_sig,d_v]
 * -> q_signal_out, q_noise_out (same shapes), k_rot [B,T,n_kv,64],
 *    lambda_out [B,T,n_sig], gate_out [B,T,n_sig,d_v]   (all fp64)
 */
int gdla_oracle_prep(const float *q_signal, const float *q_noise, const float *k_rope,
                     const float *x, const float *w_lambda, const float *gate_pre,
                     int B, int T, int n_kv, int group, int d_qk, int d_v, int d_model,
                     int pos0, double theta, double *q_signal_out, double *q_noise_out,
                     double *k_rot, double *lambda_out, double *gate_out)
{
    if (B < 0 || T < 0 || n_kv < 1 || group < 1 || d_qk < 64 || d_v < 1 || d_model < 1 ||
        pos0 < 0 || !(theta > 1.0))
        return ORACLE_BAD_ARG;
    const int n_sig = n_kv * group;
    const long n_tok = (long)B * T;
#pragma omp parallel for schedule(static)
    for (long bt = 0; bt < n_tok; ++bt) {
        const double pos = (double)(pos0 + bt % T);
        /* query heads: signal then noise */
        for (int h = 0; h < n_sig + n_kv; ++h) {
            const float *src = h < n_sig ? q_signal + (bt * n_sig + h) * d_qk
                                         : q_noise + (bt * n_kv + (h - n_sig)) * d_qk;
            double *dst = h < n_sig ? q_signal_out + (bt * n_sig + h) * d_qk
                                    : q_noise_out + (bt * n_kv + (h - n_sig)) * d_qk;
#if ORACLE_MUTANT == 16
            const int rot0 = 0;
#else
            const int rot0 = d_qk - 64;
#endif
            for (int d = 0; d < d_qk; ++d) dst[d] = src[d];
            rope64(src + rot0, pos, theta, dst + rot0);
        }
        /* the shared key, once per KV head */
        for (int j = 0; j < n_kv; ++j) {
#if ORACLE_MUTANT == 15
            if (j > 0) {
                for (int d = 0; d < 64; ++d) k_rot[(bt * n_kv + j) * 64 + d] = k_rope[bt * 64 + d];
                continue;
            }
#endif
            rope64(k_rope + bt * 64, pos, theta, k_rot + (bt * n_kv + j) * 64);
        }
        /* lambda_h = sigmoid(x_t . W^lambda[h]) */
        for (int h = 0; h < n_sig; ++h) {
            double z = 0.0;
            for (int k = 0; k < d_model; ++k)
                z += (double)x[bt * d_model + k] * (double)w_lambda[(long)h * d_model + k];
            lambda_out[bt * n_sig + h] = sigmoid(z);
        }
        for (long e = 0; e < (long)n_sig * d_v; ++e)
            gate_out[bt * n_sig * d_v + e] = sigmoid((double)gate_pre[bt * n_sig * d_v + e]);
    }
    return ORACLE_OK;
}

/* Threads for later parallel regions of this library (n >= 1). */
void gdla_oracle_set_threads(int n)
{
    if (n >= 1)
        omp_set_num_threads(n);
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
