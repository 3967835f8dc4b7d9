"""Helpers shared by the GPU parity tests: run the HIP path and the oracle on
the same bf16 inputs and compare them."""
import math

import numpy as np
import torch

import attention_gdla_prefill_amd as gdla
import oracle

# Parity bar after the gate (relative L2 over the compared elements, and max abs).
REL_L2 = 1e-2
MAX_ABS = 3e-2


def log(msg):
    print("[gdla-test] " + msg, flush=True)


def to_dev(x, device="cuda"):
    return {k: (v.to(device) if isinstance(v, torch.Tensor) else v) for k, v in x.items()}


def f32(t):
    return t.detach().float().cpu().numpy()


def compare(got, want, what=""):
    """got: bf16/float tensor or array, want: float64 array of the same shape."""
    g = got.detach().double().cpu().numpy() if isinstance(got, torch.Tensor) else np.asarray(got, np.float64)
    w = np.asarray(want, np.float64)
    assert g.shape == w.shape, (g.shape, w.shape)
    assert np.isfinite(g).all(), "%s: non-finite values in the GPU output" % what
    diff = g - w
    nw = np.linalg.norm(w)
    rel = np.linalg.norm(diff) / nw if nw > 0 else np.linalg.norm(diff)
    mabs = float(np.max(np.abs(diff))) if diff.size else 0.0
    # worst row: last dim is d_v
    rows_d = diff.reshape(-1, diff.shape[-1])
    rows_w = w.reshape(-1, w.shape[-1])
    rn = np.linalg.norm(rows_w, axis=1)
    worst = float(np.max(np.linalg.norm(rows_d, axis=1) / np.maximum(rn, 1e-30))) if rn.size else 0.0
    log("%s: rel_l2=%.3e max_abs=%.3e worst_row_rel=%.3e" % (what, rel, mabs, worst))
    assert rel <= REL_L2, "%s: rel_l2 %.3e > %.0e" % (what, rel, REL_L2)
    assert mabs <= MAX_ABS, "%s: max_abs %.3e > %.0e" % (what, mabs, MAX_ABS)
    return rel, mabs, worst


def gpu_prefill(x, window, scale=None, poison=True):
    out = None
    if poison:
        B, T, n_sig, _ = x["q_signal"].shape
        out = torch.full((B, T, n_sig, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    out = gdla.prefill(x["q_signal"], x["q_noise"], x["k"], x["v"], x["lam"], x["gate"],
                       window=window, scale=scale, out=out)
    torch.cuda.synchronize()
    return out


def oracle_prefill(x, window, scale=None):
    return oracle.prefill(f32(x["q_signal"]), f32(x["q_noise"]), f32(x["k"]), f32(x["v"]),
                          f32(x["lam"]), f32(x["gate"]), window=window, scale=scale)


def oracle_prefill_rows(x, window, rb, rt, scale=None):
    rb_t = torch.as_tensor(rb, dtype=torch.long)
    rt_t = torch.as_tensor(rt, dtype=torch.long)
    pick = lambda t: f32(t[rb_t.to(t.device), rt_t.to(t.device)])
    return oracle.prefill_rows(f32(x["k"]), f32(x["v"]), pick(x["q_signal"]), pick(x["q_noise"]),
                               pick(x["lam"]), pick(x["gate"]), rb, rt, window=window, scale=scale)


def stratified_rows(B, T, n_first, n_last, n_mid, seed):
    r = np.random.default_rng(seed)
    rows = []
    for b in range(B):
        ts = set(range(min(n_first, T))) | set(range(max(0, T - n_last), T))
        if T > n_first + n_last:
            ts |= set(r.integers(n_first, T - n_last, size=n_mid).tolist())
        rows += [(b, t) for t in sorted(ts)]
    rows = np.array(rows, dtype=np.int32)
    return rows[:, 0].copy(), rows[:, 1].copy()


def gpu_decode(d, max_len, window, scale=None):
    B = d["q_signal"].shape[0]
    out = torch.full((B, d["q_signal"].shape[1], 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    out = gdla.decode(d["q_signal"], d["q_noise"], d["k_cache"], d["v_cache"], d["cu_seqlens"],
                      max_len, d["lam"], d["gate"], window=window, scale=scale, out=out)
    torch.cuda.synchronize()
    return out


def oracle_decode(d, window, scale=None):
    return oracle.decode(f32(d["q_signal"]), f32(d["q_noise"]), f32(d["k_cache"]), f32(d["v_cache"]),
                         d["cu_seqlens"].cpu().numpy().astype(np.int32), f32(d["lam"]), f32(d["gate"]),
                         window=window, scale=scale)


def default_scale():
    return 1.0 / math.sqrt(192)


def query_tail(x, P):
    """The inputs of a prefix call: query-side tensors from position P on (the
    K/V tensors keep every row)."""
    y = dict(x)
    for k in ("q_signal", "q_noise", "lam", "gate"):
        y[k] = x[k][:, P:].contiguous()
    return y


def gpu_prefill_prefix(x, window, scale=None):
    B, Tq, n_sig, _ = x["q_signal"].shape
    out = torch.full((B, Tq, n_sig, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    out = gdla.prefill_prefix(x["q_signal"], x["q_noise"], x["k"], x["v"], x["lam"], x["gate"],
                              window=window, scale=scale, out=out)
    torch.cuda.synchronize()
    return out
