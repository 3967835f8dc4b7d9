"""The GDLA attention core for a list of query rows, written with float64
torch CPU ops -- TEST INFRASTRUCTURE ONLY (the tests, the smoke check and the
benchmark's CPU baseline may use it; the product library never does).

It computes the same plain definition as the C oracle (``gdla_oracle.c``),
for sequences too long for that one to finish in seconds (the C oracle takes
each row's dot products one by one; here the matrix products are
``torch.matmul``, a library step):

  for each listed row (b, t) and KV head j, with the visible keys
  Vis(t) = max(0, t-W+1) .. t (W = 0: 0 .. t):
    z_s = scale * q . K[b, s, j]            for s in Vis(t)
    H(q) = sum_s exp(z_s - max z) V[b, s, j] / sum_s exp(z_s - max z)
    H_S,h = H(q_signal[h]) for the signal heads h = 4j .. 4j+3
    H_N   = H(q_noise[j])
    out[h] = gate[h] * (H_S,h - lambda[h] * H_N)

Sources (web pages on the Motif 3 technical report): aitrends.kr "314B MoE
언어 모델 Motif 3의 구조와 학습 시스템", GDLA paragraph (signal and noise paths
share one KV head; D_t = H_S,t - lambda_t (.) Repeat_g(H_N,t); the element-wise
gate) and grouped-differential paragraph (g = 4; each noise head is repeated to
the signal heads of its own group); context-parallel paragraph and idailynews
(128-token sliding windows).  The readings are the C oracle's: the window
covers keys t-W+1 .. t; Repeat_g is an interleave; lambda is one scalar per
(token, signal head), used as given.

Rows are taken in position order, a few at a time, only to bound the memory
of the score matrix; no row's arithmetic depends on which others share its
chunk.  ``mutant`` (tests only) plants a numbered mistake so that the tests
can show their pins catch it; 0 is the definition.
"""
import math

import torch

# score-matrix budget per chunk (float64 elements): 32M = 256 MB
_CHUNK_ELEMS = 32 << 20


def _cpu64(t):
    t = t if isinstance(t, torch.Tensor) else torch.as_tensor(t)
    return t.detach().to("cpu", torch.float64)


def prefill_rows(k, v, q_signal_rows, q_noise_rows, lam_rows, gate_rows, row_b, row_t,
                 window=0, scale=None, mutant=0):
    """Output rows O[b_r, t_r] (float64 tensor [R, n_sig, d_v]).

    k [B, T, n_kv, d_qk], v [B, T, n_kv, d_v] (any float dtype, any device:
    widened to float64 on the CPU head by head); per-row inputs
    q_signal_rows [R, n_sig, d_qk], q_noise_rows [R, n_kv, d_qk],
    lam_rows [R, n_sig], gate_rows [R, n_sig, d_v]; row_b, row_t [R].
    """
    B, T, n_kv, d_qk = k.shape
    d_v = v.shape[3]
    qs = _cpu64(q_signal_rows)
    qn = _cpu64(q_noise_rows)
    lam = _cpu64(lam_rows)
    gate = _cpu64(gate_rows)
    R, n_sig = qs.shape[0], qs.shape[1]
    g = n_sig // n_kv
    rb = torch.as_tensor(row_b, dtype=torch.long).cpu()
    rt = torch.as_tensor(row_t, dtype=torch.long).cpu()
    if R and (rb.min() < 0 or rb.max() >= B or rt.min() < 0 or rt.max() >= T):
        raise ValueError("row index out of range")
    if scale is None:
        scale = 1.0 / math.sqrt(d_qk)
    if mutant == 4:
        scale = 1.0                                   # planted: scale forgotten
    w_eff = window + 1 if (mutant == 2 and window > 0) else window   # planted: window one too wide
    last = rt + 1 if mutant == 3 else rt              # planted: row t also sees key t+1
    first = (rt - w_eff + 1).clamp(min=0) if w_eff > 0 else torch.zeros_like(rt)
    last = last.clamp(max=T - 1)

    hs = torch.empty(R, n_sig, d_v, dtype=torch.float64)
    hn = torch.empty(R, n_kv, d_v, dtype=torch.float64)
    for b in range(B):
        mine = torch.nonzero(rb == b).flatten()
        if mine.numel() == 0:
            continue
        mine = mine[torch.argsort(rt[mine], stable=True)]
        for j in range(n_kv):
            kj = _cpu64(k[b, :, j])                    # [T, d_qk]
            vj = _cpu64(v[b, :, j])                    # [T, d_v]
            i = 0
            while i < mine.numel():
                # rows i .. e-1 of this sequence, in position order: a chunk
                # grows while its score matrix fits the budget and covers
                # little more than the keys its rows see
                e = i + 1
                seen = int(last[mine[i]] - first[mine[i]]) + 1
                while e < mine.numel():
                    lo = int(first[mine[i:e + 1]].min())
                    hi = int(last[mine[e]]) + 1
                    seen_e = seen + int(last[mine[e]] - first[mine[e]]) + 1
                    cost = (e + 1 - i) * (hi - lo)
                    if cost * (g + 1) > _CHUNK_ELEMS or cost > 1.2 * seen_e + 4096:
                        break
                    seen = seen_e
                    e += 1
                rows = mine[i:e]
                lo, hi = int(first[rows].min()), int(last[rows].max()) + 1
                keys = torch.arange(lo, hi)
                vis = (keys[None, :] >= first[rows, None]) & (keys[None, :] <= last[rows, None])   # [r, hi-lo]
                q = torch.cat([qs[rows, g * j:g * j + g], qn[rows, j:j + 1]], dim=1)               # [r, g+1, d_qk]
                z = torch.matmul(q, kj[lo:hi].T)                                                   # [r, g+1, hi-lo]
                z.mul_(scale)
                z.masked_fill_(~vis[:, None, :], float("-inf"))
                z.sub_(z.amax(dim=-1, keepdim=True)).exp_()                                        # exp(z - max z)
                h = torch.matmul(z, vj[lo:hi]) / z.sum(dim=-1, keepdim=True)                       # [r, g+1, d_v]
                hs[rows, g * j:g * j + g] = h[:, :g]
                hn[rows, j] = h[:, g]
                i = e
    if mutant == 1:                                   # planted: Repeat_g as a tile
        rep = hn[:, torch.arange(n_sig) % n_kv]
    else:
        rep = hn.repeat_interleave(g, dim=1)
    return gate * (hs - lam[..., None] * rep)
