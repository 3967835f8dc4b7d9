"""Seeded synthetic inputs for the GDLA attention core.

This module only draws random numbers and holds none of the method's
arithmetic.  Both sides of every parity check -- the HIP library and the CPU
oracle -- consume the tensors it returns, so they see bit-identical bf16
inputs.

Shapes follow Table 1 of the Motif 3 report as summarised on metalmedia
(page 2): 80 query heads over 16 KV heads, 64 signal and 16 noise heads, a
query-key head dim of 192 and a value head dim of 128; the sliding-window
layers use 128 tokens (aitrends.kr, context-parallel paragraph; idailynews).
The value distributions restate the workloads the attention core is measured
on: Q, K, V ~ N(0,1)/sqrt(192); lambda ~ U(0,1), one scalar per (token,
signal head); gate = sigmoid(N(0,1)) per (token, signal head, value dim).
All are rounded to bf16 (round-to-nearest-even, torch's conversion).

Draw order from one generator: q_signal, q_noise, k, v, lambda, gate.  Decode
sequence lengths come first, from a separate CPU generator with the same seed,
so that every device sees the same lengths.
"""
import dataclasses
import math

import torch

D_QK = 192
D_V = 128
GROUP = 4
WINDOW = 128


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    kind: str            # "prefill" or "decode"
    B: int               # batch (prefill) or number of sequences (decode)
    T: int = 0           # prefill sequence length
    n_kv: int = 16
    group: int = GROUP
    d_qk: int = D_QK
    d_v: int = D_V
    window: int = 0      # 0 = full causal, else keys t-W+1..t
    len_lo: int = 0      # decode: cached lengths ~ U{len_lo..len_hi}, new token included
    len_hi: int = 0
    prefix: int = 0      # prefill after a prefix: the queries are positions prefix .. T-1
                         # (inputs are drawn for all T positions; callers keep the query tail)

    @property
    def n_sig(self):
        return self.n_kv * self.group


# The workloads the attention core is specified on.
WORKLOADS = {
    "tiny": Workload("tiny", "prefill", B=1, T=256, n_kv=1),
    "pf_full_4k": Workload("pf_full_4k", "prefill", B=1, T=4096),
    "pf_swa_32k": Workload("pf_swa_32k", "prefill", B=2, T=32768, window=WINDOW),
    "pf_full_128k": Workload("pf_full_128k", "prefill", B=1, T=131072),
    # chunked prefill: the last 4096 tokens of a 32K sequence, full causal
    "pf_prefix_4k_32k": Workload("pf_prefix_4k_32k", "prefill", B=1, T=32768, prefix=28672),
    # one rank's share of the 32K sliding-window layer over 8 sequence-parallel
    # GPUs: 4096 tokens after the 128 rows received from the left neighbour
    "pf_swa_rank": Workload("pf_swa_rank", "prefill", B=2, T=4096 + WINDOW, window=WINDOW, prefix=WINDOW),
    "dec_full": Workload("dec_full", "decode", B=64, len_lo=8192, len_hi=65536),
    "dec_swa": Workload("dec_swa", "decode", B=64, len_lo=8192, len_hi=65536, window=WINDOW),
    # the same decodes over the latent cache (compressed KV 512 + rotary key 64)
    "dec_latent_full": Workload("dec_latent_full", "decode_latent", B=64, len_lo=8192, len_hi=65536),
    "dec_latent_swa": Workload("dec_latent_swa", "decode_latent", B=64, len_lo=8192, len_hi=65536,
                               window=WINDOW),
}


def _bf16(x):
    return x.to(torch.bfloat16)


def _draw(gen, shape, device, std):
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32) * std


def prefill_inputs(w, seed=0, device="cpu", q_std=None, k_std=None, v_std=None):
    """bf16 tensors for a prefill workload.

    Returns dict with q_signal [B,T,n_sig,d_qk], q_noise [B,T,n_kv,d_qk],
    k [B,T,n_kv,d_qk], v [B,T,n_kv,d_v], lam [B,T,n_sig], gate [B,T,n_sig,d_v].
    ``q_std``/``k_std``/``v_std`` override the N(0,1)/sqrt(d_qk) spread (the
    sharper sets used to exercise the softmax).
    """
    base = 1.0 / math.sqrt(w.d_qk)
    q_std = base if q_std is None else q_std
    k_std = base if k_std is None else k_std
    v_std = base if v_std is None else v_std
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    B, T = w.B, w.T
    out = {}
    out["q_signal"] = _bf16(_draw(gen, (B, T, w.n_sig, w.d_qk), device, q_std))
    out["q_noise"] = _bf16(_draw(gen, (B, T, w.n_kv, w.d_qk), device, q_std))
    out["k"] = _bf16(_draw(gen, (B, T, w.n_kv, w.d_qk), device, k_std))
    out["v"] = _bf16(_draw(gen, (B, T, w.n_kv, w.d_v), device, v_std))
    out["lam"] = _bf16(torch.rand((B, T, w.n_sig), generator=gen, device=device))
    out["gate"] = _bf16(torch.sigmoid(_draw(gen, (B, T, w.n_sig, w.d_v), device, 1.0)))
    return out


def decode_lengths(w, seed=0):
    """Cached lengths L_b ~ U{len_lo..len_hi} (int64, CPU), new token included."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed)
    return torch.randint(w.len_lo, w.len_hi + 1, (w.B,), generator=gen, dtype=torch.int64)


def decode_inputs(w, seed=0, device="cpu", lengths=None, q_std=None, k_std=None, v_std=None):
    """bf16 tensors for a decode workload over a packed KV cache.

    Returns dict with q_signal [B,n_sig,d_qk], q_noise [B,n_kv,d_qk],
    k_cache [total,n_kv,d_qk], v_cache [total,n_kv,d_v], cu_seqlens int32 [B+1]
    (on ``device``), lengths int64 [B] (CPU), lam [B,n_sig], gate [B,n_sig,d_v].
    """
    if lengths is None:
        lengths = decode_lengths(w, seed)
    lengths = torch.as_tensor(lengths, dtype=torch.int64).cpu()
    base = 1.0 / math.sqrt(w.d_qk)
    q_std = base if q_std is None else q_std
    k_std = base if k_std is None else k_std
    v_std = base if v_std is None else v_std
    cu = torch.zeros(lengths.numel() + 1, dtype=torch.int64)
    cu[1:] = torch.cumsum(lengths, 0)
    total = int(cu[-1])
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    B = lengths.numel()
    out = {"lengths": lengths, "cu_seqlens": cu.to(torch.int32).to(device)}
    out["q_signal"] = _bf16(_draw(gen, (B, w.n_sig, w.d_qk), device, q_std))
    out["q_noise"] = _bf16(_draw(gen, (B, w.n_kv, w.d_qk), device, q_std))
    out["k_cache"] = _bf16(_draw(gen, (total, w.n_kv, w.d_qk), device, k_std))
    out["v_cache"] = _bf16(_draw(gen, (total, w.n_kv, w.d_v), device, v_std))
    out["lam"] = _bf16(torch.rand((B, w.n_sig), generator=gen, device=device))
    out["gate"] = _bf16(torch.sigmoid(_draw(gen, (B, w.n_sig, w.d_v), device, 1.0)))
    return out


D_C = 512            # compressed KV rank (aitrends.kr, head-dimension paragraph)
D_R = 64             # rotary key dims, shared by every KV head


def latent_decode_inputs(w, seed=0, device="cpu", lengths=None, q_std=None):
    """bf16 tensors for a decode over the latent cache.

    Returns dict with q_signal [B,n_sig,192], q_noise [B,n_kv,192] (content
    128, then rotary 64), latent [total, 512+64] (compressed KV, then the
    shared rotary key), w_uk [n_kv,128,512], w_uv [n_kv,128,512],
    cu_seqlens int32 [B+1] (on ``device``), lengths int64 [B] (CPU),
    lam [B,n_sig], gate [B,n_sig,128].  The compressed KV is the output of a
    normalisation, N(0,1) per value; the up-projections are N(0,1)/sqrt(192*512),
    so the expanded keys and values have the N(0,1)/sqrt(192) spread of the
    expanded-cache workloads.  Draw order: q_signal, q_noise, latent, w_uk,
    w_uv, lambda, gate.
    """
    if lengths is None:
        lengths = decode_lengths(w, seed)
    lengths = torch.as_tensor(lengths, dtype=torch.int64).cpu()
    base = 1.0 / math.sqrt(w.d_qk)
    q_std = base if q_std is None else q_std
    cu = torch.zeros(lengths.numel() + 1, dtype=torch.int64)
    cu[1:] = torch.cumsum(lengths, 0)
    total = int(cu[-1])
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    B = lengths.numel()
    d_kc = w.d_qk - D_R
    out = {"lengths": lengths, "cu_seqlens": cu.to(torch.int32).to(device)}
    out["q_signal"] = _bf16(_draw(gen, (B, w.n_sig, w.d_qk), device, q_std))
    out["q_noise"] = _bf16(_draw(gen, (B, w.n_kv, w.d_qk), device, q_std))
    lat = _draw(gen, (total, D_C + D_R), device, 1.0)
    lat[:, D_C:] *= base
    out["latent"] = _bf16(lat)
    wstd = 1.0 / math.sqrt(w.d_qk * D_C)
    out["w_uk"] = _bf16(_draw(gen, (w.n_kv, d_kc, D_C), device, wstd))
    out["w_uv"] = _bf16(_draw(gen, (w.n_kv, w.d_v, D_C), device, wstd))
    out["lam"] = _bf16(torch.rand((B, w.n_sig), generator=gen, device=device))
    out["gate"] = _bf16(torch.sigmoid(_draw(gen, (B, w.n_sig, w.d_v), device, 1.0)))
    return out


D_MODEL = 4096          # hidden dimension (Table 1)


def prep_inputs(w, seed=0, device="cpu", d_model=D_MODEL):
    """bf16 tensors for the step ahead of the attention core, at the shapes of
    prefill workload ``w``.

    Returns dict with q_signal [B,T,n_sig,192], q_noise [B,T,n_kv,192] (before
    rotation, N(0,1)/sqrt(192)), k [B,T,n_kv,192] (content part N(0,1)/sqrt(192);
    the rotary part is overwritten by the step, drawn here too), k_rope [B,T,64]
    (the shared rotary key before rotation, N(0,1)/sqrt(192)), x [B,T,d_model]
    (hidden states, N(0,1)), w_lambda [n_sig,d_model] (N(0,1)/sqrt(d_model), so
    that x . w_lambda[h] is about N(0,1)) and gate_pre [B,T,n_sig,128] (N(0,1)).
    Draw order: q_signal, q_noise, k, k_rope, x, w_lambda, gate_pre.
    """
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    B, T = w.B, w.T
    base = 1.0 / math.sqrt(w.d_qk)
    out = {}
    out["q_signal"] = _bf16(_draw(gen, (B, T, w.n_sig, w.d_qk), device, base))
    out["q_noise"] = _bf16(_draw(gen, (B, T, w.n_kv, w.d_qk), device, base))
    out["k"] = _bf16(_draw(gen, (B, T, w.n_kv, w.d_qk), device, base))
    out["k_rope"] = _bf16(_draw(gen, (B, T, 64), device, base))
    out["x"] = _bf16(_draw(gen, (B, T, d_model), device, 1.0))
    out["w_lambda"] = _bf16(_draw(gen, (w.n_sig, d_model), device, 1.0 / math.sqrt(d_model)))
    out["gate_pre"] = _bf16(_draw(gen, (B, T, w.n_sig, w.d_v), device, 1.0))
    return out
