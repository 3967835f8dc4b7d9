// gdla_api.hip -- the extern "C" entry points declared in include/gdla.h:
// host-side argument checks (before any HIP call), then the kernel launches.
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>

#include "gdla.h"
#include "gdla_launch.h"

namespace {

thread_local char g_last_error[256] = "";

int fail(int code, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return code;
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

struct Range {
    const char *name;
    uintptr_t lo, hi;
};

bool overlaps(const Range &a, const Range &b) { return a.lo < b.hi && b.lo < a.hi; }

int check_head_shape(int n_kv, int group, int d_qk, int d_v) {
    if (n_kv < 1 || group < 1 || d_qk < 1 || d_v < 1)
        return fail(GDLA_ERR_INVALID_ARG, "n_kv, group, d_qk, d_v must be >= 1 (got %d, %d, %d, %d)",
                    n_kv, group, d_qk, d_v);
    if (group != 4 || d_qk != 192 || d_v != 128)
        return fail(GDLA_ERR_UNSUPPORTED,
                    "this build implements group=4, d_qk=192, d_v=128 (got %d, %d, %d)", group, d_qk, d_v);
    return GDLA_OK;
}

int check_scale_window(float scale, int window) {
    if (!std::isfinite(scale) || !(scale > 0.f))
        return fail(GDLA_ERR_INVALID_ARG, "softmax_scale must be finite and > 0 (got %g)", (double)scale);
    if (window < 0) return fail(GDLA_ERR_INVALID_ARG, "window must be >= 0 (got %d)", window);
    return GDLA_OK;
}

}  // namespace

extern "C" int gdla_abi_version(void) { return 1; }

extern "C" const char *gdla_status_string(int status) {
    switch (status) {
        case GDLA_OK: return "GDLA_OK";
        case GDLA_ERR_INVALID_ARG: return "GDLA_ERR_INVALID_ARG: invalid argument";
        case GDLA_ERR_UNSUPPORTED: return "GDLA_ERR_UNSUPPORTED: head shape not implemented";
        case GDLA_ERR_MISALIGNED: return "GDLA_ERR_MISALIGNED: tensor pointer not 16-byte aligned";
        case GDLA_ERR_WORKSPACE: return "GDLA_ERR_WORKSPACE: decode workspace missing or too small";
        case GDLA_ERR_HIP: return "GDLA_ERR_HIP: HIP runtime error";
        default: return "GDLA: unknown status";
    }
}

extern "C" const char *gdla_last_error(void) { return g_last_error; }

extern "C" int gdla_prefill_prefix(const void *q_signal, const void *q_noise, const void *k,
                                   const void *v, const void *lambda_, const void *gate, void *out,
                                   int B, int T_q, int P, int n_kv, int group, int d_qk, int d_v,
                                   int window, float softmax_scale, void *stream) {
    g_last_error[0] = 0;
    if (B < 0 || T_q < 0 || P < 0)
        return fail(GDLA_ERR_INVALID_ARG, "B, T_q and P must be >= 0 (got %d, %d, %d)", B, T_q, P);
    if (int rc = check_head_shape(n_kv, group, d_qk, d_v)) return rc;
    if (int rc = check_scale_window(softmax_scale, window)) return rc;
    if (B == 0 || T_q == 0) return GDLA_OK;

    const void *ptrs[7] = {q_signal, q_noise, k, v, lambda_, gate, out};
    const char *names[7] = {"q_signal", "q_noise", "k", "v", "lambda", "gate", "out"};
    for (int i = 0; i < 7; ++i) {
        if (!ptrs[i]) return fail(GDLA_ERR_INVALID_ARG, "%s is NULL", names[i]);
        if (!aligned(ptrs[i], 16)) return fail(GDLA_ERR_MISALIGNED, "%s is not 16-byte aligned", names[i]);
    }
    const long double Tk = (long double)P + T_q;
    const long double n_sig = (long double)n_kv * group;
    if ((long double)B * Tk * n_sig * d_qk * 2 >= 4.6e18L)
        return fail(GDLA_ERR_INVALID_ARG, "tensor sizes exceed the 2^62-byte limit");
    if (Tk >= 2147483647.0L - 64) return fail(GDLA_ERR_INVALID_ARG, "P + T_q must be < 2^31 - 64");
    if (gdla::prefill_grid_blocks(B, T_q, P, n_kv) >= (1L << 31))
        return fail(GDLA_ERR_INVALID_ARG, "B * n_kv * (query tiles) must be < 2^31");
    if ((Tk + 64) * n_kv * d_qk * 2 >= 2147483648.0L)
        return fail(GDLA_ERR_UNSUPPORTED,
                    "one sequence's K rows must span < 2^31 bytes ((P+T_q+64)*n_kv*d_qk*2)");

    const uintptr_t rq = (uintptr_t)B * (uintptr_t)T_q;
    const uintptr_t rk = (uintptr_t)B * ((uintptr_t)P + (uintptr_t)T_q);
    const uintptr_t ns = (uintptr_t)n_kv * group;
    const Range in[6] = {
        {"q_signal", (uintptr_t)q_signal, (uintptr_t)q_signal + rq * ns * d_qk * 2},
        {"q_noise", (uintptr_t)q_noise, (uintptr_t)q_noise + rq * n_kv * d_qk * 2},
        {"k", (uintptr_t)k, (uintptr_t)k + rk * n_kv * d_qk * 2},
        {"v", (uintptr_t)v, (uintptr_t)v + rk * n_kv * d_v * 2},
        {"lambda", (uintptr_t)lambda_, (uintptr_t)lambda_ + rq * ns * 2},
        {"gate", (uintptr_t)gate, (uintptr_t)gate + rq * ns * d_v * 2}};
    const Range o = {"out", (uintptr_t)out, (uintptr_t)out + rq * ns * d_v * 2};
    for (const Range &x : in)
        if (overlaps(o, x)) return fail(GDLA_ERR_INVALID_ARG, "out overlaps %s", x.name);

    hipError_t e = gdla::launch_prefill(q_signal, q_noise, k, v, lambda_, gate, out, B, T_q, P, n_kv,
                                        window, softmax_scale, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(GDLA_ERR_HIP, "prefill launch: %s", hipGetErrorString(e));
    return GDLA_OK;
}

extern "C" int gdla_prefill(const void *q_signal, const void *q_noise, const void *k, const void *v,
                            const void *lambda_, const void *gate, void *out, int B, int T, int n_kv,
                            int group, int d_qk, int d_v, int window, float softmax_scale,
                            void *stream) {
    if (T < 0) {
        g_last_error[0] = 0;
        return fail(GDLA_ERR_INVALID_ARG, "B and T must be >= 0 (got %d, %d)", B, T);
    }
    return gdla_prefill_prefix(q_signal, q_noise, k, v, lambda_, gate, out, B, T, 0, n_kv, group,
                               d_qk, d_v, window, softmax_scale, stream);
}

extern "C" size_t gdla_decode_workspace_size(int B, int n_kv, int max_seqlen_k, int window) {
    if (B < 1 || n_kv < 1 || max_seqlen_k < 1 || window < 0) return 0;
    return gdla::decode_workspace_bytes(B, n_kv, gdla::decode_splits(max_seqlen_k, window));
}

namespace {

// Checks shared by gdla_decode and gdla_decode_noalloc.  `workspace` is the
// area the split partials go to (the caller's, or the library's scratch);
// with `own_workspace` false its size and alignment are the caller's to
// check.  Returns the status; on GDLA_OK, n_split and need are set.
int check_decode(const void *q_signal, const void *q_noise, const void *k_cache, const void *v_cache,
                 const int32_t *cu_seqlens_k, int max_seqlen_k, const void *lambda_, const void *gate,
                 const void *out, const void *workspace, size_t workspace_bytes, bool own_workspace, int B,
                 int n_kv, int group, int d_qk, int d_v, int window, float softmax_scale, int &n_split,
                 size_t &need) {
    if (B < 0 || B > 65535) return fail(GDLA_ERR_INVALID_ARG, "B must be in [0, 65535] (got %d)", B);
    if (int rc = check_head_shape(n_kv, group, d_qk, d_v)) return rc;
    if (n_kv > 65535) return fail(GDLA_ERR_INVALID_ARG, "n_kv must be <= 65535 (got %d)", n_kv);
    if (int rc = check_scale_window(softmax_scale, window)) return rc;
    n_split = 1;
    need = 0;
    if (B == 0) return GDLA_OK;
    if (max_seqlen_k < 1) return fail(GDLA_ERR_INVALID_ARG, "max_seqlen_k must be >= 1 (got %d)", max_seqlen_k);

    const void *ptrs[7] = {q_signal, q_noise, k_cache, v_cache, lambda_, gate, out};
    const char *names[7] = {"q_signal", "q_noise", "k_cache", "v_cache", "lambda", "gate", "out"};
    for (int i = 0; i < 7; ++i) {
        if (!ptrs[i]) return fail(GDLA_ERR_INVALID_ARG, "%s is NULL", names[i]);
        if (!aligned(ptrs[i], 16)) return fail(GDLA_ERR_MISALIGNED, "%s is not 16-byte aligned", names[i]);
    }
    if (!cu_seqlens_k) return fail(GDLA_ERR_INVALID_ARG, "cu_seqlens_k is NULL");
    if (!aligned(cu_seqlens_k, 4)) return fail(GDLA_ERR_MISALIGNED, "cu_seqlens_k is not 4-byte aligned");

    n_split = gdla::decode_splits(max_seqlen_k, window);
    need = gdla::decode_workspace_bytes(B, n_kv, n_split);
    if (need > 0 && own_workspace) {
        if (!workspace) return fail(GDLA_ERR_WORKSPACE, "workspace is NULL, %zu bytes needed", need);
        if (workspace_bytes < need)
            return fail(GDLA_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, need);
        if (!aligned(workspace, 16)) return fail(GDLA_ERR_MISALIGNED, "workspace is not 16-byte aligned");
    }
    // the inputs whose extent the call knows (the caches' row count is not an
    // argument), the output and the workspace the split kernel writes
    const uintptr_t ns = (uintptr_t)n_kv * group;
    const Range o = {"out", (uintptr_t)out, (uintptr_t)out + (uintptr_t)B * ns * d_v * 2};
    const Range w = {"workspace", (uintptr_t)workspace, (uintptr_t)workspace + need};
    const Range in[5] = {
        {"q_signal", (uintptr_t)q_signal, (uintptr_t)q_signal + (uintptr_t)B * ns * d_qk * 2},
        {"q_noise", (uintptr_t)q_noise, (uintptr_t)q_noise + (uintptr_t)B * n_kv * d_qk * 2},
        {"lambda", (uintptr_t)lambda_, (uintptr_t)lambda_ + (uintptr_t)B * ns * 2},
        {"gate", (uintptr_t)gate, (uintptr_t)gate + (uintptr_t)B * ns * d_v * 2},
        {"cu_seqlens_k", (uintptr_t)cu_seqlens_k, (uintptr_t)cu_seqlens_k + ((uintptr_t)B + 1) * 4}};
    for (const Range &x : in) {
        if (overlaps(o, x)) return fail(GDLA_ERR_INVALID_ARG, "out overlaps %s", x.name);
        if (own_workspace && need > 0 && overlaps(w, x))
            return fail(GDLA_ERR_INVALID_ARG, "workspace overlaps %s", x.name);
    }
    if (own_workspace && need > 0 && overlaps(o, w)) return fail(GDLA_ERR_INVALID_ARG, "out overlaps workspace");
    return GDLA_OK;
}

}  // namespace

extern "C" int gdla_decode(const void *q_signal, const void *q_noise, const void *k_cache,
                           const void *v_cache, const int32_t *cu_seqlens_k, int max_seqlen_k,
                           const void *lambda_, const void *gate, void *out, void *workspace,
                           size_t workspace_bytes, int B, int n_kv, int group, int d_qk, int d_v,
                           int window, float softmax_scale, void *stream) {
    g_last_error[0] = 0;
    int n_split = 1;
    size_t need = 0;
    if (int rc = check_decode(q_signal, q_noise, k_cache, v_cache, cu_seqlens_k, max_seqlen_k, lambda_, gate, out,
                              workspace, workspace_bytes, true, B, n_kv, group, d_qk, d_v, window, softmax_scale,
                              n_split, need))
        return rc;
    if (B == 0) return GDLA_OK;
    hipError_t e = gdla::launch_decode(q_signal, q_noise, k_cache, v_cache, cu_seqlens_k, lambda_,
                                       gate, out, workspace, B, n_kv, n_split, window, softmax_scale,
                                       static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(GDLA_ERR_HIP, "decode launch: %s", hipGetErrorString(e));
    return GDLA_OK;
}

extern "C" size_t gdla_decode_noalloc_max_scratch(void) { return gdla::DECODE_NOALLOC_SCRATCH_BYTES; }

extern "C" int gdla_decode_noalloc(const void *q_signal, const void *q_noise, const void *k_cache,
                                   const void *v_cache, const int32_t *cu_seqlens_k, int max_seqlen_k,
                                   const void *lambda_, const void *gate, void *out, int B, int n_kv, int group,
                                   int d_qk, int d_v, int window, float softmax_scale, void *stream) {
    g_last_error[0] = 0;
    int n_split = 1;
    size_t need = 0;
    if (int rc = check_decode(q_signal, q_noise, k_cache, v_cache, cu_seqlens_k, max_seqlen_k, lambda_, gate, out,
                              nullptr, 0, false, B, n_kv, group, d_qk, d_v, window, softmax_scale, n_split, need))
        return rc;
    if (B == 0) return GDLA_OK;
    if (need > gdla::DECODE_NOALLOC_SCRATCH_BYTES)
        return fail(GDLA_ERR_WORKSPACE,
                    "the split partials need %zu bytes, more than the %zu-byte scratch of gdla_decode_noalloc "
                    "(use gdla_decode with a workspace, or fewer sequences or KV heads per call)",
                    need, gdla::DECODE_NOALLOC_SCRATCH_BYTES);
    void *scratch = nullptr;
    if (need > 0) {
        hipError_t e = gdla::decode_noalloc_scratch(&scratch);
        if (e != hipSuccess) return fail(GDLA_ERR_HIP, "decode scratch lookup: %s", hipGetErrorString(e));
        const Range w = {"scratch", (uintptr_t)scratch, (uintptr_t)scratch + need};
        const Range o = {"out", (uintptr_t)out, (uintptr_t)out + (uintptr_t)B * n_kv * group * d_v * 2};
        if (overlaps(o, w)) return fail(GDLA_ERR_INVALID_ARG, "out overlaps the library's scratch");
    }
    hipError_t e = gdla::launch_decode(q_signal, q_noise, k_cache, v_cache, cu_seqlens_k, lambda_,
                                       gate, out, scratch, B, n_kv, n_split, window, softmax_scale,
                                       static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(GDLA_ERR_HIP, "decode launch: %s", hipGetErrorString(e));
    return GDLA_OK;
}

extern "C" size_t gdla_decode_latent_workspace_size(int B, int n_kv, int max_seqlen_k, int window) {
    if (B < 1 || n_kv < 1 || max_seqlen_k < 1 || window < 0) return 0;
    return gdla::latent_workspace_bytes(B, n_kv, gdla::latent_splits(max_seqlen_k, window));
}

extern "C" int gdla_decode_latent(const void *q_signal, const void *q_noise, const void *latent_cache,
                                  const int32_t *cu_seqlens_k, int max_seqlen_k, const void *w_uk,
                                  const void *w_uv, const void *lambda_, const void *gate, void *out,
                                  void *workspace, size_t workspace_bytes, int B, int n_kv, int group,
                                  int d_c, int d_r, int d_v, int window, float softmax_scale,
                                  void *stream) {
    g_last_error[0] = 0;
    if (B < 0 || B > 65535) return fail(GDLA_ERR_INVALID_ARG, "B must be in [0, 65535] (got %d)", B);
    if (n_kv < 1 || group < 1 || d_c < 1 || d_r < 0 || d_v < 1)
        return fail(GDLA_ERR_INVALID_ARG, "n_kv, group, d_c, d_v must be >= 1 and d_r >= 0");
    if (group != 4 || d_c != 512 || d_r != 64 || d_v != 128)
        return fail(GDLA_ERR_UNSUPPORTED,
                    "this build implements group=4, d_c=512, d_r=64, d_v=128 (got %d, %d, %d, %d)",
                    group, d_c, d_r, d_v);
    if (n_kv > 13107) return fail(GDLA_ERR_INVALID_ARG, "n_kv must be <= 13107 (got %d)", n_kv);
    if (int rc = check_scale_window(softmax_scale, window)) return rc;
    if (B == 0) return GDLA_OK;
    if (max_seqlen_k < 1) return fail(GDLA_ERR_INVALID_ARG, "max_seqlen_k must be >= 1 (got %d)", max_seqlen_k);

    const void *ptrs[8] = {q_signal, q_noise, latent_cache, w_uk, w_uv, lambda_, gate, out};
    const char *names[8] = {"q_signal", "q_noise", "latent_cache", "w_uk", "w_uv", "lambda", "gate", "out"};
    for (int i = 0; i < 8; ++i) {
        if (!ptrs[i]) return fail(GDLA_ERR_INVALID_ARG, "%s is NULL", names[i]);
        if (!aligned(ptrs[i], 16)) return fail(GDLA_ERR_MISALIGNED, "%s is not 16-byte aligned", names[i]);
    }
    if (!cu_seqlens_k) return fail(GDLA_ERR_INVALID_ARG, "cu_seqlens_k is NULL");
    if (!aligned(cu_seqlens_k, 4)) return fail(GDLA_ERR_MISALIGNED, "cu_seqlens_k is not 4-byte aligned");
    if ((long double)max_seqlen_k * (d_c + d_r) * 2 >= 4294967296.0L)
        return fail(GDLA_ERR_UNSUPPORTED, "one sequence's latent rows must span < 2^32 bytes");

    const int n_split = gdla::latent_splits(max_seqlen_k, window);
    const size_t need = gdla::latent_workspace_bytes(B, n_kv, n_split);
    if (!workspace) return fail(GDLA_ERR_WORKSPACE, "workspace is NULL, %zu bytes needed", need);
    if (workspace_bytes < need)
        return fail(GDLA_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, need);
    if (!aligned(workspace, 256)) return fail(GDLA_ERR_MISALIGNED, "workspace is not 256-byte aligned");

    const uintptr_t ns = (uintptr_t)n_kv * group;
    const Range o = {"out", (uintptr_t)out, (uintptr_t)out + (uintptr_t)B * ns * d_v * 2};
    const Range w = {"workspace", (uintptr_t)workspace, (uintptr_t)workspace + need};
    const int d_qk = d_v + d_r;                  // the content part of a query is d_v = 128 values
    const Range in[7] = {
        {"q_signal", (uintptr_t)q_signal, (uintptr_t)q_signal + (uintptr_t)B * ns * d_qk * 2},
        {"q_noise", (uintptr_t)q_noise, (uintptr_t)q_noise + (uintptr_t)B * n_kv * d_qk * 2},
        {"w_uk", (uintptr_t)w_uk, (uintptr_t)w_uk + (uintptr_t)n_kv * 128 * d_c * 2},
        {"w_uv", (uintptr_t)w_uv, (uintptr_t)w_uv + (uintptr_t)n_kv * d_v * d_c * 2},
        {"lambda", (uintptr_t)lambda_, (uintptr_t)lambda_ + (uintptr_t)B * ns * 2},
        {"gate", (uintptr_t)gate, (uintptr_t)gate + (uintptr_t)B * ns * d_v * 2},
        {"cu_seqlens_k", (uintptr_t)cu_seqlens_k, (uintptr_t)cu_seqlens_k + ((uintptr_t)B + 1) * 4}};
    for (const Range &x : in) {
        if (overlaps(o, x)) return fail(GDLA_ERR_INVALID_ARG, "out overlaps %s", x.name);
        if (overlaps(w, x)) return fail(GDLA_ERR_INVALID_ARG, "workspace overlaps %s", x.name);
    }
    if (overlaps(o, w)) return fail(GDLA_ERR_INVALID_ARG, "out overlaps workspace");

    hipError_t e = gdla::launch_decode_latent(q_signal, q_noise, latent_cache, cu_seqlens_k, w_uk, w_uv,
                                              lambda_, gate, out, workspace, B, n_kv, n_split, window,
                                              softmax_scale, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(GDLA_ERR_HIP, "latent decode launch: %s", hipGetErrorString(e));
    return GDLA_OK;
}

extern "C" int gdla_prep(void *q_signal, void *q_noise, const void *k_rope, void *k, const void *x,
                         const void *w_lambda, void *lambda_out, const void *gate_pre, void *gate_out,
                         int B, int T, int n_kv, int group, int d_qk, int d_v, int d_model, int pos0,
                         float rope_theta, void *stream) {
    g_last_error[0] = 0;
    if (B < 0 || T < 0 || pos0 < 0)
        return fail(GDLA_ERR_INVALID_ARG, "B, T and pos0 must be >= 0 (got %d, %d, %d)", B, T, pos0);
    if (int rc = check_head_shape(n_kv, group, d_qk, d_v)) return rc;
    if (d_model < 1) return fail(GDLA_ERR_INVALID_ARG, "d_model must be >= 1 (got %d)", d_model);
    if (d_model % 32 != 0)
        return fail(GDLA_ERR_UNSUPPORTED, "this build needs d_model to be a multiple of 32 (got %d)", d_model);
    if (!std::isfinite(rope_theta) || !(rope_theta > 1.f))
        return fail(GDLA_ERR_INVALID_ARG, "rope_theta must be finite and > 1 (got %g)", (double)rope_theta);
    if ((long)pos0 + T > 2147483647L) return fail(GDLA_ERR_INVALID_ARG, "pos0 + T must be < 2^31");
    if (B == 0 || T == 0) return GDLA_OK;

    void *ptrs[9] = {q_signal, q_noise, const_cast<void *>(k_rope), k, const_cast<void *>(x),
                     const_cast<void *>(w_lambda), lambda_out, const_cast<void *>(gate_pre), gate_out};
    const char *names[9] = {"q_signal", "q_noise", "k_rope", "k", "x", "w_lambda", "lambda_out", "gate_pre",
                            "gate_out"};
    for (int i = 0; i < 9; ++i) {
        if (!ptrs[i]) return fail(GDLA_ERR_INVALID_ARG, "%s is NULL", names[i]);
        if (!aligned(ptrs[i], 16)) return fail(GDLA_ERR_MISALIGNED, "%s is not 16-byte aligned", names[i]);
    }
    const long double n_tok = (long double)B * T;
    const long double ns = (long double)n_kv * group;
    if (n_tok * ((long double)d_model + ns * d_qk + ns * d_v) * 2 >= 4.6e18L)
        return fail(GDLA_ERR_INVALID_ARG, "tensor sizes exceed the 2^62-byte limit");
    if (gdla::prep_grid_blocks((long)B * T) >= (1L << 31))
        return fail(GDLA_ERR_INVALID_ARG, "B * T / 16 must be < 2^31");

    const uintptr_t nt = (uintptr_t)B * (uintptr_t)T, s = (uintptr_t)n_kv * group;
    auto R = [](const char *n, const void *p, uintptr_t bytes) {
        return Range{n, (uintptr_t)p, (uintptr_t)p + bytes};
    };
    const Range outs[5] = {R("q_signal", q_signal, nt * s * d_qk * 2), R("q_noise", q_noise, nt * n_kv * d_qk * 2),
                           R("k", k, nt * n_kv * d_qk * 2), R("lambda_out", lambda_out, nt * s * 2),
                           R("gate_out", gate_out, nt * s * d_v * 2)};
    const Range ins[4] = {R("k_rope", k_rope, nt * 64 * 2), R("x", x, nt * d_model * 2),
                          R("w_lambda", w_lambda, s * d_model * 2), R("gate_pre", gate_pre, nt * s * d_v * 2)};
    for (int i = 0; i < 5; ++i) {
        for (int j = i + 1; j < 5; ++j)
            if (overlaps(outs[i], outs[j]))
                return fail(GDLA_ERR_INVALID_ARG, "%s overlaps %s", outs[i].name, outs[j].name);
        for (const Range &in : ins) {
            // the gate may be computed in place
            if (i == 4 && in.lo == outs[4].lo && in.hi == outs[4].hi) continue;
            if (overlaps(outs[i], in)) return fail(GDLA_ERR_INVALID_ARG, "%s overlaps %s", outs[i].name, in.name);
        }
    }

    hipError_t e = gdla::launch_prep(q_signal, q_noise, k_rope, k, x, w_lambda, lambda_out, gate_pre, gate_out, B,
                                     T, n_kv, d_model, pos0, rope_theta, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(GDLA_ERR_HIP, "prep launch: %s", hipGetErrorString(e));
    return GDLA_OK;
}

extern "C" size_t gdla_prefill_backward_workspace_size(int B, int T, int n_kv) {
    if (B < 0 || T < 0 || n_kv < 1) return 0;
    return gdla::backward_workspace_bytes(B, T, n_kv);
}

extern "C" int gdla_prefill_backward(const void *q_signal, const void *q_noise, const void *k, const void *v,
                                     const void *lambda_, const void *gate, const void *d_out, void *dq_signal,
                                     void *dq_noise, void *dk, void *dv, void *dlambda, void *dgate,
                                     void *workspace, size_t workspace_bytes, int B, int T, int n_kv, int group,
                                     int d_qk, int d_v, int window, float softmax_scale, void *stream) {
    g_last_error[0] = 0;
    if (B < 0 || T < 0) return fail(GDLA_ERR_INVALID_ARG, "B and T must be >= 0 (got %d, %d)", B, T);
    if (int rc = check_head_shape(n_kv, group, d_qk, d_v)) return rc;
    if (int rc = check_scale_window(softmax_scale, window)) return rc;
    if (B == 0 || T == 0) return GDLA_OK;
    if (B > 65535 || n_kv > 65535) return fail(GDLA_ERR_INVALID_ARG, "B and n_kv must be <= 65535");
    if (T > 65535 * 64) return fail(GDLA_ERR_INVALID_ARG, "T must be <= 65535 * 64 (the 64-token tiles of a grid dimension)");

    const void *ptrs[13] = {q_signal, q_noise, k, v, lambda_, gate, d_out, dq_signal, dq_noise, dk, dv, dlambda,
                            dgate};
    const char *names[13] = {"q_signal", "q_noise", "k", "v", "lambda", "gate", "d_out", "dq_signal", "dq_noise",
                             "dk", "dv", "dlambda", "dgate"};
    for (int i = 0; i < 13; ++i) {
        if (!ptrs[i]) return fail(GDLA_ERR_INVALID_ARG, "%s is NULL", names[i]);
        if (!aligned(ptrs[i], 16)) return fail(GDLA_ERR_MISALIGNED, "%s is not 16-byte aligned", names[i]);
    }
    const long double ns = (long double)n_kv * group;
    if ((long double)B * T * ns * d_qk * 2 >= 4.6e18L)
        return fail(GDLA_ERR_INVALID_ARG, "tensor sizes exceed the 2^62-byte limit");
    if ((long double)T >= 2147483647.0L - 64) return fail(GDLA_ERR_INVALID_ARG, "T must be < 2^31 - 64");
    if (gdla::prefill_grid_blocks(B, T, 0, n_kv) >= (1L << 31))
        return fail(GDLA_ERR_INVALID_ARG, "B * n_kv * (query tiles) must be < 2^31");
    if (((long double)T + 64) * n_kv * d_qk * 2 >= 2147483648.0L)
        return fail(GDLA_ERR_UNSUPPORTED, "one sequence's K rows must span < 2^31 bytes ((T+64)*n_kv*d_qk*2)");
    const size_t need = gdla::backward_workspace_bytes(B, T, n_kv);
    if (!workspace) return fail(GDLA_ERR_WORKSPACE, "workspace is NULL, %zu bytes needed", need);
    if (workspace_bytes < need)
        return fail(GDLA_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, need);
    if (!aligned(workspace, 256)) return fail(GDLA_ERR_MISALIGNED, "workspace is not 256-byte aligned");

    const uintptr_t rows = (uintptr_t)B * (uintptr_t)T, s = (uintptr_t)n_kv * group;
    auto R = [](const char *n, const void *p, uintptr_t bytes) {
        return Range{n, (uintptr_t)p, (uintptr_t)p + bytes};
    };
    const Range ins[7] = {R("q_signal", q_signal, rows * s * d_qk * 2), R("q_noise", q_noise, rows * n_kv * d_qk * 2),
                          R("k", k, rows * n_kv * d_qk * 2), R("v", v, rows * n_kv * d_v * 2),
                          R("lambda", lambda_, rows * s * 2), R("gate", gate, rows * s * d_v * 2),
                          R("d_out", d_out, rows * s * d_v * 2)};
    const Range outs[7] = {R("dq_signal", dq_signal, rows * s * d_qk * 2),
                           R("dq_noise", dq_noise, rows * n_kv * d_qk * 2), R("dk", dk, rows * n_kv * d_qk * 2),
                           R("dv", dv, rows * n_kv * d_v * 2), R("dlambda", dlambda, rows * s * 2),
                           R("dgate", dgate, rows * s * d_v * 2), R("workspace", workspace, need)};
    for (int i = 0; i < 7; ++i) {
        for (int j = i + 1; j < 7; ++j)
            if (overlaps(outs[i], outs[j])) return fail(GDLA_ERR_INVALID_ARG, "%s overlaps %s", outs[i].name, outs[j].name);
        for (const Range &in : ins)
            if (overlaps(outs[i], in)) return fail(GDLA_ERR_INVALID_ARG, "%s overlaps %s", outs[i].name, in.name);
    }

    hipError_t e = gdla::launch_backward(q_signal, q_noise, k, v, lambda_, gate, d_out, dq_signal, dq_noise, dk, dv,
                                         dlambda, dgate, workspace, B, T, n_kv, window, softmax_scale,
                                         static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(GDLA_ERR_HIP, "backward launch: %s", hipGetErrorString(e));
    return GDLA_OK;
}
