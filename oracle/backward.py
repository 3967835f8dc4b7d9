"""CPU oracle for the gradients of the GDLA attention core -- TEST
INFRASTRUCTURE ONLY (the tests, the smoke check and the benchmark's CPU
baseline may use it; the product library never does).

The forward is the plain definition written with float64 torch CPU ops (no
tiling, no online softmax), and the gradients are torch's automatic
differentiation of it.  Sources: aitrends.kr "314B MoE 언어 모델 Motif 3의
구조와 학습 시스템", GDLA paragraphs (per KV head j, the signal heads of its
group and noise head j attend with the same K_j and V_j;
D = H_S - lambda (.) Repeat_g(H_N); then the element-wise gate) and
grouped-differential paragraph (g = 4); the window reading (keys t-W+1 .. t)
and the interleaved Repeat_g are the same readings as the C oracle's.

It is pinned independently of itself by the tests: its forward equals the C
oracle's on random inputs, its gradients equal central finite differences of
that forward, and the gradients satisfy identities of the softmax (the key
gradients of each query row sum to zero; the value gradients sum to the
output gradients).

``forward`` takes a ``mutant`` switch (tests only) that plants a mistake, so
that the tests can show the pins catch it; 0 is the definition.
"""
import math

import torch


def _mask(T, window, device="cpu"):
    t = torch.arange(T, device=device)
    vis = t[None, :] <= t[:, None]                       # key s <= query t
    if window > 0:
        vis &= (t[:, None] - t[None, :]) < window        # keys t-W+1 .. t
    return vis


def forward(q_signal, q_noise, k, v, lam, gate, window=0, scale=None, parts=False, mutant=0):
    """out [B,T,n_sig,d_v] for float64 tensors q_signal [B,T,n_sig,d_qk],
    q_noise [B,T,n_kv,d_qk], k [B,T,n_kv,d_qk], v [B,T,n_kv,d_v],
    lam [B,T,n_sig], gate [B,T,n_sig,d_v].  With parts=True also returns
    (H_S, H_N)."""
    B, T, n_kv, d_qk = k.shape
    n_sig = q_signal.shape[2]
    g = n_sig // n_kv
    if scale is None:
        scale = 1.0 / math.sqrt(d_qk)
    if mutant == 3:
        scale = 1.0
    vis = _mask(T, window + (1 if mutant == 2 and window > 0 else 0))

    def attend(q, kk, vv):
        # q [B,T,H,d] against one KV head's kk [B,T,d], vv [B,T,d_v]
        s = torch.einsum("bthd,bsd->bhts", q, kk) * scale
        s = s.masked_fill(~vis, float("-inf"))
        p = torch.softmax(s, dim=-1)
        return torch.einsum("bhts,bsd->bthd", p, vv)

    hs = torch.cat([attend(q_signal[:, :, g * j:g * j + g], k[:, :, j], v[:, :, j]) for j in range(n_kv)], dim=2)
    hn = torch.cat([attend(q_noise[:, :, j:j + 1], k[:, :, j], v[:, :, j]) for j in range(n_kv)], dim=2)
    rep = hn.repeat(1, 1, g, 1) if mutant == 1 else hn.repeat_interleave(g, dim=2)
    out = gate * (hs - lam[..., None] * rep)
    return (out, hs, hn) if parts else out


NAMES = ("q_signal", "q_noise", "k", "v", "lam", "gate")


def backward(q_signal, q_noise, k, v, lam, gate, d_out, window=0, scale=None):
    """Gradients of sum(d_out * out) with respect to the six inputs, as a dict
    of float64 tensors keyed by NAMES.  Inputs may be any float tensors; they
    are widened to float64 on the CPU."""
    xs = [t.detach().to("cpu", torch.float64).requires_grad_(True)
          for t in (q_signal, q_noise, k, v, lam, gate)]
    out = forward(*xs, window=window, scale=scale)
    grads = torch.autograd.grad(out, xs, d_out.detach().to("cpu", torch.float64))
    return dict(zip(NAMES, grads))
