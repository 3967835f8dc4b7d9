/*
 * gdla.h -- C ABI of the GDLA attention core on AMD Instinct MI355X (gfx950).
 *
 * Grouped Differential Latent Attention (GDLA), as the Motif 3 technical
 * report describes it (aitrends.kr, "314B MoE 언어 모델 Motif 3의 구조와 학습
 * 시스템", GDLA and grouped-differential paragraphs; shapes from metalmedia,
 * Table 1): every KV head j serves one group of `group` = 4 signal query heads
 * (4j .. 4j+3) and one noise query head (j).  Both paths share the KV head's
 * K (query-key dim 192) and V (value dim 128), and each query head runs causal
 * softmax attention over it -- full causal, or a sliding window of W keys
 * (the report's hybrid layers use W = 128; aitrends.kr context-parallel
 * paragraph, idailynews).  The library then forms
 *     D[t,h,:] = H_S[t,h,:] - lambda[t,h] * H_N[t, h/4, :]
 * (the noise output repeated to the 4 signal heads of its group) and applies
 * the element-wise output gate,
 *     out[t,h,:] = gate[t,h,:] * D[t,h,:].
 * The output projection that follows in the model is not part of this
 * library.  With a window W >= 1 a query at position t sees keys
 * max(0, t-W+1) .. t; with W = 0 it sees 0 .. t.
 *
 * Conventions shared by every entry point:
 *   - Every tensor pointer is a DEVICE pointer to a dense, row-major array
 *     (last dimension fastest) of bf16 values, unless stated otherwise, and
 *     must be 16-byte aligned.  The caller owns all memory; the library
 *     allocates nothing, keeps no pointer after the call returns, and holds no
 *     mutable global state besides a per-thread error-detail string (and the
 *     per-GPU scratch array of gdla_decode_noalloc, described there).
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Work is enqueued on it and the call returns without waiting; the caller
 *     synchronises before reading `out`.
 *   - Arguments are checked on the host before any HIP call.  A rejected call
 *     returns a nonzero status, launches nothing and leaves `out` untouched.
 *     gdla_last_error() gives a one-line reason for the last nonzero status
 *     returned on the calling thread.
 *   - Values are used as given: lambda is not clamped and the scale is not
 *     altered.  Arithmetic: bf16 products accumulated in fp32, softmax in
 *     fp32, the combine and gate in fp32, one rounding to bf16 (nearest-even)
 *     on the final store.
 *   - This build supports group = 4, d_qk = 192, d_v = 128 and any
 *     n_kv >= 1; other head shapes return GDLA_ERR_UNSUPPORTED.
 *   - Two environment variables, read by the prefill entry points at every
 *     call, exist for testing: GDLA_PREFILL_GRID (a positive integer) caps the
 *     number of persistent workgroups, GDLA_PREFILL_RUN_LEN sets the query
 *     tiles per work item of a window of up to 129 keys.  Results do not
 *     depend on either.
 */
#ifndef GDLA_H
#define GDLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned (as int) by every entry point. */
enum gdla_status {
    GDLA_OK = 0,
    GDLA_ERR_INVALID_ARG = 1,   /* null pointer, negative size, non-finite scale, ...   */
    GDLA_ERR_UNSUPPORTED = 2,   /* head shape outside what this build implements       */
    GDLA_ERR_MISALIGNED = 3,    /* a tensor pointer is not 16-byte aligned             */
    GDLA_ERR_WORKSPACE = 4,     /* decode workspace missing or smaller than required   */
    GDLA_ERR_HIP = 5            /* the HIP runtime reported an error at launch         */
};

/* Version of this ABI (incremented on any incompatible change). */
int gdla_abi_version(void);

/* Static, human-readable name of a status code. */
const char *gdla_status_string(int status);

/* Reason for the last nonzero status returned on this thread ("" if none). */
const char *gdla_last_error(void);

/*
 * gdla_prefill -- attention core for every position of B sequences of T
 * tokens (prefill / training-forward shape).
 *
 *   q_signal [B, T, n_kv*group, d_qk]  signal queries (post-RoPE); head h reads KV head h/group
 *   q_noise  [B, T, n_kv, d_qk]        noise queries; head j reads KV head j
 *   k        [B, T, n_kv, d_qk]        keys (post-RoPE)
 *   v        [B, T, n_kv, d_v]         values
 *   lambda_  [B, T, n_kv*group]        one coefficient per (token, signal head)
 *   gate     [B, T, n_kv*group, d_v]   output gate, already through its sigmoid
 *   out      [B, T, n_kv*group, d_v]   result; every element is written; must
 *                                      not overlap any input
 *   window        0 = full causal, W >= 1 = sliding window of W keys
 *   softmax_scale multiplies q.k before the softmax (callers usually pass
 *                 1/sqrt(d_qk)); must be finite
 *
 * B = 0 or T = 0 is a valid empty call: GDLA_OK, nothing launched.
 * Limits: B*T*n_kv*group*d_v < 2^62; B*n_kv*ceil(T/64) < 2^31; one
 * sequence's K rows must span less than 2^31 bytes, (T+64)*n_kv*d_qk*2 < 2^31
 * (T = 131072 allows n_kv up to 42), else GDLA_ERR_UNSUPPORTED.
 */
int gdla_prefill(const void *q_signal, const void *q_noise, const void *k, const void *v,
                 const void *lambda_, const void *gate, void *out,
                 int B, int T, int n_kv, int group, int d_qk, int d_v,
                 int window, float softmax_scale, void *stream);

/*
 * gdla_prefill_prefix -- the same attention core for T_q new tokens that follow
 * a prefix of P tokens whose K and V are already there: chunked prefill, or one
 * rank's share of a sequence-parallel layer together with the K/V rows it
 * received from its left neighbour (the digest's window-aware context
 * parallelism exchanges exactly the last W rows: aitrends.kr, context-parallel
 * paragraph).  Query row i sits at position P + i.
 *
 *   q_signal [B, T_q, n_kv*group, d_qk]   queries of the new tokens
 *   q_noise  [B, T_q, n_kv, d_qk]
 *   k        [B, P + T_q, n_kv, d_qk]     rows 0 .. P-1: the prefix; P .. P+T_q-1: the new tokens
 *   v        [B, P + T_q, n_kv, d_v]
 *   lambda_  [B, T_q, n_kv*group]
 *   gate     [B, T_q, n_kv*group, d_v]
 *   out      [B, T_q, n_kv*group, d_v]   every element written; no overlap with inputs
 *   window   0 = full causal: row i sees keys 0 .. P+i; W >= 1: keys max(0, P+i-W+1) .. P+i
 *
 * Row i of the result equals row P + i of gdla_prefill over the whole P + T_q
 * tokens.  gdla_prefill(..., T, ...) is gdla_prefill_prefix(..., T, 0, ...).
 * B = 0 or T_q = 0 is a valid empty call.  Limits as for gdla_prefill with
 * P + T_q in place of T; P < 0 is GDLA_ERR_INVALID_ARG.
 */
int gdla_prefill_prefix(const void *q_signal, const void *q_noise, const void *k, const void *v,
                        const void *lambda_, const void *gate, void *out,
                        int B, int T_q, int P, int n_kv, int group, int d_qk, int d_v,
                        int window, float softmax_scale, void *stream);

/*
 * gdla_decode_workspace_size -- bytes of device workspace gdla_decode needs
 * for B sequences, n_kv KV heads, cached lengths up to max_seqlen_k and the
 * given window.  0 means no workspace is needed (a single pass suffices).
 * Returns 0 as well for invalid arguments (gdla_decode then rejects them).
 */
size_t gdla_decode_workspace_size(int B, int n_kv, int max_seqlen_k, int window);

/*
 * gdla_decode -- attention core for one new token per sequence over a packed
 * KV cache (autoregressive decode).  The cache holds the expanded per-head
 * K and V; the report's KV path expands the compressed KV into 16 KV heads
 * and shares one KV state between the signal and noise paths (aitrends.kr,
 * GDLA paragraph; metalmedia, Table 1).
 *
 *   q_signal     [B, n_kv*group, d_qk]
 *   q_noise      [B, n_kv, d_qk]
 *   k_cache      [total_k, n_kv, d_qk]   sequence b owns rows cu[b] .. cu[b+1]-1
 *   v_cache      [total_k, n_kv, d_v]
 *   cu_seqlens_k DEVICE int32 [B+1], nondecreasing, 4-byte aligned.  The
 *                length L_b = cu[b+1]-cu[b] already includes the new token
 *                (the caller appends its K/V first); the query sits at
 *                position L_b-1 and sees keys max(0, L_b-W) .. L_b-1.  A
 *                sequence with L_b <= 0 gets an all-zero output row.
 *   max_seqlen_k host-side upper bound on L_b; it sizes the split of the
 *                cache across workgroups (any L_b is still computed
 *                correctly, only less evenly split, if it is exceeded)
 *   lambda_      [B, n_kv*group]
 *   gate         [B, n_kv*group, d_v]
 *   out          [B, n_kv*group, d_v]   every element written; no overlap with inputs
 *   workspace    device scratch of at least
 *                gdla_decode_workspace_size(B, n_kv, max_seqlen_k, window)
 *                bytes (may be NULL when that size is 0); contents on entry
 *                are ignored; calls sharing one workspace must be ordered on
 *                one stream
 *
 * B = 0 is a valid empty call.
 */
int gdla_decode(const void *q_signal, const void *q_noise, const void *k_cache,
                const void *v_cache, const int32_t *cu_seqlens_k, int max_seqlen_k,
                const void *lambda_, const void *gate, void *out,
                void *workspace, size_t workspace_bytes,
                int B, int n_kv, int group, int d_qk, int d_v,
                int window, float softmax_scale, void *stream);

/*
 * gdla_decode_noalloc -- gdla_decode for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same arguments without the workspace, the same
 * kernels and the same result, bit for bit.  The split partials go to a
 * scratch array inside the library instead: one per GPU, of
 * gdla_decode_noalloc_max_scratch() bytes (96 MiB), held from the library's
 * first use on that GPU until the process ends.  The call itself allocates
 * nothing (no hipMalloc, hipFree or allocating library routine); its first
 * call on a GPU looks up that GPU's scratch address.
 *
 * A call whose partials would need more than that
 * (gdla_decode_workspace_size(B, n_kv, max_seqlen_k, window) bytes) returns
 * GDLA_ERR_WORKSPACE and launches nothing; 64 sequences of up to 65,536
 * cached tokens over 16 KV heads need 82 MiB.  Every call on one GPU shares
 * its scratch and the scratch keeps the last call's contents: calls that
 * overlap on one GPU (unordered streams) race, so order them on one stream.
 * Arguments, limits and errors otherwise as for gdla_decode.
 */
size_t gdla_decode_noalloc_max_scratch(void);
int gdla_decode_noalloc(const void *q_signal, const void *q_noise, const void *k_cache,
                        const void *v_cache, const int32_t *cu_seqlens_k, int max_seqlen_k,
                        const void *lambda_, const void *gate, void *out,
                        int B, int n_kv, int group, int d_qk, int d_v,
                        int window, float softmax_scale, void *stream);

/*
 * gdla_decode_latent_workspace_size -- bytes of device workspace
 * gdla_decode_latent needs (never 0: it always holds the absorbed queries).
 * Returns 0 for invalid arguments (gdla_decode_latent then rejects them).
 */
size_t gdla_decode_latent_workspace_size(int B, int n_kv, int max_seqlen_k, int window);

/*
 * gdla_decode_latent -- the decode of gdla_decode over a latent KV cache: the
 * cache holds, per token, the normalised compressed KV c (d_c = 512 values)
 * followed by the decoupled rotary key k^R (d_r = 64 values), shared by every
 * KV head, instead of the expanded per-head K and V (aitrends.kr, GDLA and
 * head-dimension paragraphs: the compressed KV of rank 512 is normalised once
 * and expanded to the 16 KV heads; the rotary key is shared by all of them).
 * KV head j's keys and values are
 *     K_j[s] = [ W_uk[j] c_s ; k^R_s ]   (128 + 64 = 192 values)
 *     V_j[s] =   W_uv[j] c_s             (128 values)
 * and the result equals gdla_decode over those K and V.  The library does not
 * form them: it folds W_uk into the queries and W_uv into the output, so each
 * cache row (1,152 bytes) is read once for all query heads.
 *
 *   q_signal     [B, n_kv*group, 192]    content part (128) first, then rotary (64)
 *   q_noise      [B, n_kv, 192]
 *   latent_cache [total_k, d_c + d_r]    sequence b owns rows cu[b] .. cu[b+1]-1
 *   cu_seqlens_k, max_seqlen_k           as for gdla_decode
 *   w_uk         [n_kv, 128, d_c]        key up-projection: k^C = w_uk[j] c
 *   w_uv         [n_kv, d_v, d_c]        value up-projection: v = w_uv[j] c
 *   lambda_      [B, n_kv*group]
 *   gate         [B, n_kv*group, d_v]
 *   out          [B, n_kv*group, d_v]    every element written; no overlap with inputs
 *   workspace    device scratch of at least
 *                gdla_decode_latent_workspace_size(B, n_kv, max_seqlen_k, window)
 *                bytes, 256-byte aligned; contents on entry are ignored;
 *                calls sharing one workspace must be ordered on one stream
 *
 * The absorbed queries are rounded to bf16 before the scores (the only
 * rounding the expanded path does not have).  B = 0 is a valid empty call.
 * This build supports group = 4, d_c = 512, d_r = 64, d_v = 128; other
 * shapes return GDLA_ERR_UNSUPPORTED.
 */
int gdla_decode_latent(const void *q_signal, const void *q_noise, const void *latent_cache,
                       const int32_t *cu_seqlens_k, int max_seqlen_k, const void *w_uk,
                       const void *w_uv, const void *lambda_, const void *gate, void *out,
                       void *workspace, size_t workspace_bytes,
                       int B, int n_kv, int group, int d_c, int d_r, int d_v,
                       int window, float softmax_scale, void *stream);

/*
 * gdla_prep -- the step ahead of gdla_prefill / gdla_prefill_prefix, fused
 * into one pass over the tokens (aitrends.kr, GDLA paragraph: the query path
 * gives a content and a rotary query, the KV path a compressed KV and a
 * decoupled rotary key, lambda_t = sigmoid(x_t W^lambda), and a query-based
 * element-wise gate follows the subtraction; head-dimension paragraph: the
 * rotary component is 64 values and the rotary key is shared by every KV
 * head; metalmedia, Table 1: attention with output gating).
 *
 *   q_signal   [B, T, n_kv*group, d_qk]  in/out: values 128..191 of each head (the
 *                                        rotary part) rotated in place, 0..127 untouched
 *   q_noise    [B, T, n_kv, d_qk]        in/out, as q_signal
 *   k_rope     [B, T, 64]                the shared rotary key before rotation
 *   k          [B, T, n_kv, d_qk]        out: values 128..191 of every KV head receive
 *                                        the rotated shared key; 0..127 untouched
 *   x          [B, T, d_model]           hidden states
 *   w_lambda   [n_kv*group, d_model]     lambda projection (row h serves signal head h)
 *   lambda_out [B, T, n_kv*group]        out: sigmoid(x_t . w_lambda[h])
 *   gate_pre   [B, T, n_kv*group, d_v]   the output gate's pre-activations
 *   gate_out   [B, T, n_kv*group, d_v]   out: sigmoid(gate_pre); may be gate_pre itself
 *   pos0       position of token 0 (token t of every sequence sits at pos0 + t;
 *              pass P for the new tokens of gdla_prefill_prefix)
 *   rope_theta base of the rotary frequencies (10000 in the original rotary
 *              embedding)
 *
 * Rotation: the original rotary embedding on adjacent pairs, for i = 0..31
 *     (r[2i], r[2i+1]) <- (r[2i] c - r[2i+1] s, r[2i] s + r[2i+1] c),
 *     c, s = cos, sin(pos * rope_theta^(-2i/64));
 * angles and their sines in fp64, the rotation in fp32, results rounded to
 * bf16 (round to nearest even); lambda's dot products accumulate in fp32.
 * Outputs must not overlap each other or the inputs (except gate_out ==
 * gate_pre).  B = 0 or T = 0 is a valid empty call.  This build supports
 * group = 4, d_qk = 192, d_v = 128 and d_model a multiple of 32; other shapes
 * return GDLA_ERR_UNSUPPORTED.
 */
int gdla_prep(void *q_signal, void *q_noise, const void *k_rope, void *k, const void *x,
              const void *w_lambda, void *lambda_out, const void *gate_pre, void *gate_out,
              int B, int T, int n_kv, int group, int d_qk, int d_v, int d_model, int pos0,
              float rope_theta, void *stream);

/*
 * gdla_prefill_backward_workspace_size -- bytes of device workspace
 * gdla_prefill_backward needs (0 for invalid arguments).
 */
size_t gdla_prefill_backward_workspace_size(int B, int T, int n_kv);

/*
 * gdla_prefill_backward -- gradients of gdla_prefill (P = 0) with respect to
 * its six inputs, given d_out, the gradient of a loss with respect to out.
 * The derivatives of the attention core (aitrends.kr, GDLA paragraphs: per KV
 * head j, signal heads 4j..4j+3 and noise head j attend with K_j, V_j;
 * D = H_S - lambda (.) Repeat_4(H_N); out = gate (.) D):
 *     dgate = d_out (.) D,  dD = gate (.) d_out,
 *     dlambda_h = -sum_d dD_h H_N,   dH_S = dD,   dH_N,j = -sum_{h in j} lambda_h dD_h,
 * then per head, with P its softmax weights and delta = rowsum(dH (.) H):
 *     dV_j += P^T dH,  dS = P (.) (dH V_j^T - delta),  dQ = scale dS K_j,
 *     dK_j += scale dS^T Q.
 * The call recomputes the forward first (the pages' long-context training
 * recomputes activations operator by operator), so it needs only the forward's
 * inputs.  Arguments as for gdla_prefill; the outputs
 *   dq_signal [B, T, n_kv*group, d_qk], dq_noise [B, T, n_kv, d_qk],
 *   dk [B, T, n_kv, d_qk], dv [B, T, n_kv, d_v], dlambda [B, T, n_kv*group],
 *   dgate [B, T, n_kv*group, d_v]
 * are bf16, every element written; none may overlap an input, another output
 * or the workspace.  workspace: device scratch of at least
 * gdla_prefill_backward_workspace_size(B, T, n_kv) bytes, 256-byte aligned,
 * contents ignored; calls sharing one must be ordered on one stream.
 * Products are bf16 with fp32 accumulation; P and dS are rounded to bf16
 * before the products that take them.  B = 0 or T = 0 is a valid empty call;
 * B and n_kv must be <= 65535 and T <= 65535 * 64.  Shape support as for
 * gdla_prefill.
 */
int gdla_prefill_backward(const void *q_signal, const void *q_noise, const void *k, const void *v,
                          const void *lambda_, const void *gate, const void *d_out, void *dq_signal,
                          void *dq_noise, void *dk, void *dv, void *dlambda, void *dgate,
                          void *workspace, size_t workspace_bytes, int B, int T, int n_kv, int group,
                          int d_qk, int d_v, int window, float softmax_scale, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GDLA_H */
