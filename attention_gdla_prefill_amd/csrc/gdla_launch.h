// gdla_launch.h -- host-side launchers of the gfx950 kernels (internal to the
// library; the public surface is include/gdla.h).  Arguments are assumed
// validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdla {


// Prefill of Tq query rows per sequence at positions P .. P+Tq-1 over P+Tq key rows.
// save_hs / save_hn / save_lse non-null (with P = 0): also write the per-head
// outputs and the log2-sum-exp of every head's softmax row
hipError_t launch_prefill(const void *qs, const void *qn, const void *k, const void *v,
                          const void *lam, const void *gate, void *out, int B, int Tq, int P, int n_kv,
                          int window, float scale, hipStream_t stream, void *save_hs = nullptr,
                          void *save_hn = nullptr, float *save_lse = nullptr);
// Query tiles of one (sequence, KV head) times B * n_kv.
long prefill_grid_blocks(int B, int Tq, int P, int n_kv);

// Number of cache splits (workgroups per (sequence, KV head)) for decode.
int decode_splits(int max_seqlen_k, int window);
// Workspace bytes for the split partials (0 when decode_splits() == 1).
size_t decode_workspace_bytes(int B, int n_kv, int n_split);

hipError_t launch_decode(const void *qs, const void *qn, const void *kc, const void *vc,
                         const int32_t *cu_seqlens, const void *lam, const void *gate, void *out,
                         void *workspace, int B, int n_kv, int n_split, int window, float scale,
                         hipStream_t stream);

// Largest split-partials area gdla_decode_noalloc can hold (its device
// scratch array), and the current device's address of that array (looked up
// on the first call on each device).
constexpr size_t DECODE_NOALLOC_SCRATCH_BYTES = (size_t)96 << 20;
hipError_t decode_noalloc_scratch(void **ptr);

// Backward: workspace bytes, launch (the saving forward and the gradient kernels).
size_t backward_workspace_bytes(int B, int T, int n_kv);
hipError_t launch_backward(const void *qs, const void *qn, const void *k, const void *v, const void *lam,
                           const void *gate, const void *dout, void *dqs, void *dqn, void *dk, void *dv,
                           void *dlam, void *dgate, void *workspace, int B, int T, int n_kv, int window,
                           float scale, hipStream_t stream);

long prep_grid_blocks(long n_tok);
hipError_t launch_prep(void *q_signal, void *q_noise, const void *k_rope, void *k, const void *x,
                       const void *w_lambda, void *lambda_out, const void *gate_pre, void *gate_out,
                       int B, int T, int n_kv, int d_model, int pos0, float rope_theta, hipStream_t stream);

// Latent-cache decode: splits per sequence, workspace bytes, launch.
int latent_splits(int max_seqlen_k, int window);
size_t latent_workspace_bytes(int B, int n_kv, int n_split);
hipError_t launch_decode_latent(const void *qs, const void *qn, const void *lat, const int32_t *cu,
                                const void *wuk, const void *wuv, const void *lam, const void *gate,
                                void *out, void *workspace, int B, int n_kv, int n_split, int window,
                                float scale, hipStream_t stream);

}  // namespace gdla
