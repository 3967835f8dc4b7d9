"""Python binding of the GDLA attention core: argument marshalling only.

Every step of the computation runs in the HIP kernels behind include/gdla.h;
these functions check tensor metadata, pick the current HIP stream and call
the C ABI through ctypes.  Tensors are torch bf16 tensors on a ROCm device.

With the environment variable GDLA_SYNC_CHECK=1 every call waits for its
kernels before returning, so that an asynchronous HIP error (a fault inside
a kernel) is raised by the call that caused it rather than by a later one.
"""
import ctypes
import math

import torch

from . import _lib

D_QK, D_V, GROUP = 192, 128, 4


def _stream_ptr(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check(t, name, shape, dtype=torch.bfloat16):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s (got %s)" % (name, dtype, t.dtype))
    if t.device.type != "cuda":
        raise ValueError("%s must be on a ROCm device (got %s)" % (name, t.device))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s (got %s)" % (name, tuple(shape), tuple(t.shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def prefill(q_signal, q_noise, k, v, lam, gate, window=0, scale=None, out=None):
    """GDLA attention core over every position of a [B, T] batch.

    q_signal [B,T,4*n_kv,192], q_noise [B,T,n_kv,192], k [B,T,n_kv,192],
    v [B,T,n_kv,128], lam [B,T,4*n_kv], gate [B,T,4*n_kv,128], all bf16.
    window 0 = full causal, W >= 1 = keys t-W+1..t.  Returns out
    [B,T,4*n_kv,128] bf16, enqueued on the current stream.
    """
    B, T, n_kv, d_qk = k.shape
    n_sig = n_kv * GROUP
    _check(q_signal, "q_signal", (B, T, n_sig, D_QK))
    _check(q_noise, "q_noise", (B, T, n_kv, D_QK))
    _check(k, "k", (B, T, n_kv, D_QK))
    _check(v, "v", (B, T, n_kv, D_V))
    _check(lam, "lam", (B, T, n_sig))
    _check(gate, "gate", (B, T, n_sig, D_V))
    if out is None:
        out = torch.empty((B, T, n_sig, D_V), dtype=torch.bfloat16, device=k.device)
    _check(out, "out", (B, T, n_sig, D_V))
    if scale is None:
        scale = 1.0 / math.sqrt(D_QK)
    lib = _lib.load()
    _lib.check(lib.gdla_prefill(
        q_signal.data_ptr(), q_noise.data_ptr(), k.data_ptr(), v.data_ptr(), lam.data_ptr(),
        gate.data_ptr(), out.data_ptr(), B, T, n_kv, GROUP, D_QK, D_V, int(window),
        float(scale), _stream_ptr(k.device)))
    _lib.after_launch(k.device)
    return out


def prefill_prefix(q_signal, q_noise, k, v, lam, gate, window=0, scale=None, out=None):
    """The attention core for T_q new tokens after a prefix already in K/V.

    q_signal [B,T_q,4*n_kv,192], q_noise [B,T_q,n_kv,192], lam [B,T_q,4*n_kv],
    gate [B,T_q,4*n_kv,128]; k [B,P+T_q,n_kv,192] and v [B,P+T_q,n_kv,128]
    hold the P prefix rows first.  Query row i sits at position P + i.
    Returns out [B,T_q,4*n_kv,128] bf16, enqueued on the current stream.
    """
    B, Tk, n_kv, d_qk = k.shape
    Tq = q_signal.shape[1]
    P = Tk - Tq
    if P < 0:
        raise ValueError("k has %d rows per sequence, fewer than the %d queries" % (Tk, Tq))
    n_sig = n_kv * GROUP
    _check(q_signal, "q_signal", (B, Tq, n_sig, D_QK))
    _check(q_noise, "q_noise", (B, Tq, n_kv, D_QK))
    _check(k, "k", (B, Tk, n_kv, D_QK))
    _check(v, "v", (B, Tk, n_kv, D_V))
    _check(lam, "lam", (B, Tq, n_sig))
    _check(gate, "gate", (B, Tq, n_sig, D_V))
    if out is None:
        out = torch.empty((B, Tq, n_sig, D_V), dtype=torch.bfloat16, device=k.device)
    _check(out, "out", (B, Tq, n_sig, D_V))
    if scale is None:
        scale = 1.0 / math.sqrt(D_QK)
    lib = _lib.load()
    _lib.check(lib.gdla_prefill_prefix(
        q_signal.data_ptr(), q_noise.data_ptr(), k.data_ptr(), v.data_ptr(), lam.data_ptr(),
        gate.data_ptr(), out.data_ptr(), B, Tq, P, n_kv, GROUP, D_QK, D_V, int(window),
        float(scale), _stream_ptr(k.device)))
    _lib.after_launch(k.device)
    return out


def decode_workspace_size(B, n_kv, max_seqlen_k, window=0):
    return int(_lib.load().gdla_decode_workspace_size(B, n_kv, max_seqlen_k, int(window)))


def decode(q_signal, q_noise, k_cache, v_cache, cu_seqlens, max_seqlen_k, lam, gate,
           window=0, scale=None, out=None, workspace=None):
    """GDLA attention core for one new token per sequence over a packed KV cache.

    q_signal [B,4*n_kv,192], q_noise [B,n_kv,192], k_cache [total,n_kv,192],
    v_cache [total,n_kv,128], cu_seqlens int32 [B+1] (device; lengths include
    the new token), lam [B,4*n_kv], gate [B,4*n_kv,128].  Returns out
    [B,4*n_kv,128] bf16.  The workspace (uint8 device tensor) is allocated
    here if not given.
    """
    total, n_kv, _ = k_cache.shape
    B = q_signal.shape[0]
    n_sig = n_kv * GROUP
    _check(q_signal, "q_signal", (B, n_sig, D_QK))
    _check(q_noise, "q_noise", (B, n_kv, D_QK))
    _check(k_cache, "k_cache", (total, n_kv, D_QK))
    _check(v_cache, "v_cache", (total, n_kv, D_V))
    _check(cu_seqlens, "cu_seqlens", (B + 1,), dtype=torch.int32)
    _check(lam, "lam", (B, n_sig))
    _check(gate, "gate", (B, n_sig, D_V))
    if out is None:
        out = torch.empty((B, n_sig, D_V), dtype=torch.bfloat16, device=k_cache.device)
    _check(out, "out", (B, n_sig, D_V))
    if scale is None:
        scale = 1.0 / math.sqrt(D_QK)
    need = decode_workspace_size(B, n_kv, max_seqlen_k, window) if B > 0 else 0
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=k_cache.device)
    lib = _lib.load()
    _lib.check(lib.gdla_decode(
        q_signal.data_ptr(), q_noise.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
        cu_seqlens.data_ptr(), int(max_seqlen_k), lam.data_ptr(), gate.data_ptr(),
        out.data_ptr(), workspace.data_ptr(), workspace.numel(), B, n_kv, GROUP, D_QK, D_V,
        int(window), float(scale), _stream_ptr(k_cache.device)))
    _lib.after_launch(k_cache.device)
    return out


def decode_noalloc_max_scratch():
    """Bytes of the library's per-GPU scratch that decode_noalloc uses."""
    return int(_lib.load().gdla_decode_noalloc_max_scratch())


def decode_noalloc(q_signal, q_noise, k_cache, v_cache, cu_seqlens, max_seqlen_k, lam, gate,
                   window=0, scale=None, out=None):
    """decode() without a workspace: the split partials go to the library's
    own per-GPU scratch (gdla_decode_noalloc).  With `out` given the call
    allocates nothing; calls on one GPU must be ordered on one stream."""
    total, n_kv, _ = k_cache.shape
    B = q_signal.shape[0]
    n_sig = n_kv * GROUP
    _check(q_signal, "q_signal", (B, n_sig, D_QK))
    _check(q_noise, "q_noise", (B, n_kv, D_QK))
    _check(k_cache, "k_cache", (total, n_kv, D_QK))
    _check(v_cache, "v_cache", (total, n_kv, D_V))
    _check(cu_seqlens, "cu_seqlens", (B + 1,), dtype=torch.int32)
    _check(lam, "lam", (B, n_sig))
    _check(gate, "gate", (B, n_sig, D_V))
    if out is None:
        out = torch.empty((B, n_sig, D_V), dtype=torch.bfloat16, device=k_cache.device)
    _check(out, "out", (B, n_sig, D_V))
    if scale is None:
        scale = 1.0 / math.sqrt(D_QK)
    lib = _lib.load()
    _lib.check(lib.gdla_decode_noalloc(
        q_signal.data_ptr(), q_noise.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
        cu_seqlens.data_ptr(), int(max_seqlen_k), lam.data_ptr(), gate.data_ptr(),
        out.data_ptr(), B, n_kv, GROUP, D_QK, D_V, int(window), float(scale), _stream_ptr(k_cache.device)))
    _lib.after_launch(k_cache.device)
    return out


D_C, D_R = 512, 64


def decode_latent_workspace_size(B, n_kv, max_seqlen_k, window=0):
    return int(_lib.load().gdla_decode_latent_workspace_size(B, n_kv, max_seqlen_k, int(window)))


def decode_latent(q_signal, q_noise, latent_cache, cu_seqlens, max_seqlen_k, w_uk, w_uv, lam, gate,
                  window=0, scale=None, out=None, workspace=None):
    """Decode over a latent KV cache (compressed KV + shared rotary key per token).

    q_signal [B,4*n_kv,192], q_noise [B,n_kv,192] (content 128, then rotary 64),
    latent_cache [total,576], cu_seqlens int32 [B+1] (device), w_uk [n_kv,128,512],
    w_uv [n_kv,128,512], lam [B,4*n_kv], gate [B,4*n_kv,128].  Returns out
    [B,4*n_kv,128] bf16; equal to decode() over K_j = [w_uk[j] c ; k^R],
    V_j = w_uv[j] c.  The workspace (uint8 device tensor) is allocated here if
    not given.
    """
    total = latent_cache.shape[0]
    n_kv = w_uk.shape[0]
    B = q_signal.shape[0]
    n_sig = n_kv * GROUP
    _check(q_signal, "q_signal", (B, n_sig, D_QK))
    _check(q_noise, "q_noise", (B, n_kv, D_QK))
    _check(latent_cache, "latent_cache", (total, D_C + D_R))
    _check(cu_seqlens, "cu_seqlens", (B + 1,), dtype=torch.int32)
    _check(w_uk, "w_uk", (n_kv, D_QK - D_R, D_C))
    _check(w_uv, "w_uv", (n_kv, D_V, D_C))
    _check(lam, "lam", (B, n_sig))
    _check(gate, "gate", (B, n_sig, D_V))
    if out is None:
        out = torch.empty((B, n_sig, D_V), dtype=torch.bfloat16, device=latent_cache.device)
    _check(out, "out", (B, n_sig, D_V))
    if scale is None:
        scale = 1.0 / math.sqrt(D_QK)
    need = decode_latent_workspace_size(B, n_kv, max_seqlen_k, window) if B > 0 else 0
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=latent_cache.device)
    lib = _lib.load()
    _lib.check(lib.gdla_decode_latent(
        q_signal.data_ptr(), q_noise.data_ptr(), latent_cache.data_ptr(), cu_seqlens.data_ptr(),
        int(max_seqlen_k), w_uk.data_ptr(), w_uv.data_ptr(), lam.data_ptr(), gate.data_ptr(),
        out.data_ptr(), workspace.data_ptr(), workspace.numel(), B, n_kv, GROUP, D_C, D_R, D_V,
        int(window), float(scale), _stream_ptr(latent_cache.device)))
    _lib.after_launch(latent_cache.device)
    return out


def prep(q_signal, q_noise, k_rope, k, x, w_lambda, gate_pre, pos0=0, rope_theta=10000.0,
         lam_out=None, gate_out=None):
    """The step ahead of the attention core, in one launch.

    Rotates the rotary part (values 128..191) of every head of q_signal
    [B,T,4*n_kv,192] and q_noise [B,T,n_kv,192] in place, writes the rotated
    shared key k_rope [B,T,64] into the rotary part of every KV head of k
    [B,T,n_kv,192], and returns (lam [B,T,4*n_kv], gate [B,T,4*n_kv,128]) with
    lam = sigmoid(x @ w_lambda^T) for x [B,T,d_model], w_lambda [4*n_kv,
    d_model], and gate = sigmoid(gate_pre).  gate_out may be gate_pre itself.
    Token t sits at position pos0 + t.  All bf16, enqueued on the current stream.
    """
    B, T, n_kv, _ = k.shape
    n_sig = n_kv * GROUP
    d_model = x.shape[-1]
    _check(q_signal, "q_signal", (B, T, n_sig, D_QK))
    _check(q_noise, "q_noise", (B, T, n_kv, D_QK))
    _check(k_rope, "k_rope", (B, T, 64))
    _check(k, "k", (B, T, n_kv, D_QK))
    _check(x, "x", (B, T, d_model))
    _check(w_lambda, "w_lambda", (n_sig, d_model))
    _check(gate_pre, "gate_pre", (B, T, n_sig, D_V))
    if lam_out is None:
        lam_out = torch.empty((B, T, n_sig), dtype=torch.bfloat16, device=k.device)
    if gate_out is None:
        gate_out = torch.empty((B, T, n_sig, D_V), dtype=torch.bfloat16, device=k.device)
    _check(lam_out, "lam_out", (B, T, n_sig))
    _check(gate_out, "gate_out", (B, T, n_sig, D_V))
    lib = _lib.load()
    _lib.check(lib.gdla_prep(
        q_signal.data_ptr(), q_noise.data_ptr(), k_rope.data_ptr(), k.data_ptr(), x.data_ptr(),
        w_lambda.data_ptr(), lam_out.data_ptr(), gate_pre.data_ptr(), gate_out.data_ptr(), B, T, n_kv,
        GROUP, D_QK, D_V, d_model, int(pos0), float(rope_theta), _stream_ptr(k.device)))
    _lib.after_launch(k.device)
    return lam_out, gate_out


def prefill_backward_workspace_size(B, T, n_kv):
    return int(_lib.load().gdla_prefill_backward_workspace_size(B, T, n_kv))


def prefill_backward(q_signal, q_noise, k, v, lam, gate, d_out, window=0, scale=None, workspace=None):
    """Gradients of prefill(q_signal, q_noise, k, v, lam, gate, window, scale)
    with respect to its six inputs, given d_out [B,T,4*n_kv,128] (the
    gradient of a loss with respect to its output).  The forward is recomputed
    inside.  Returns a dict of bf16 tensors keyed q_signal, q_noise, k, v, lam,
    gate (each of its input's shape); enqueued on the current stream.  The
    workspace (uint8 device tensor) is allocated here if not given."""
    B, T, n_kv, _ = k.shape
    n_sig = n_kv * GROUP
    _check(q_signal, "q_signal", (B, T, n_sig, D_QK))
    _check(q_noise, "q_noise", (B, T, n_kv, D_QK))
    _check(k, "k", (B, T, n_kv, D_QK))
    _check(v, "v", (B, T, n_kv, D_V))
    _check(lam, "lam", (B, T, n_sig))
    _check(gate, "gate", (B, T, n_sig, D_V))
    _check(d_out, "d_out", (B, T, n_sig, D_V))
    if scale is None:
        scale = 1.0 / math.sqrt(D_QK)
    need = prefill_backward_workspace_size(B, T, n_kv)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=k.device)
    grads = {name: torch.empty_like(t) for name, t in
             (("q_signal", q_signal), ("q_noise", q_noise), ("k", k), ("v", v), ("lam", lam), ("gate", gate))}
    lib = _lib.load()
    _lib.check(lib.gdla_prefill_backward(
        q_signal.data_ptr(), q_noise.data_ptr(), k.data_ptr(), v.data_ptr(), lam.data_ptr(), gate.data_ptr(),
        d_out.data_ptr(), grads["q_signal"].data_ptr(), grads["q_noise"].data_ptr(), grads["k"].data_ptr(),
        grads["v"].data_ptr(), grads["lam"].data_ptr(), grads["gate"].data_ptr(), workspace.data_ptr(),
        workspace.numel(), B, T, n_kv, GROUP, D_QK, D_V, int(window), float(scale), _stream_ptr(k.device)))
    _lib.after_launch(k.device)
    return grads
