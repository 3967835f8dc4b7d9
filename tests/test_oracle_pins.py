"""Pins for the CPU oracle, each against something other than the oracle itself.

The pages (Motif 3 report summaries; the GDLA equations are on aitrends.kr,
"314B MoE 언어 모델 Motif 3의 구조와 학습 시스템") print no worked example, so
the pins are:
  * a hand-derived closed-form example (tests/golden/closed_form_T3.txt);
  * special cases that reduce to a library routine: lambda = 0 is plain
    softmax attention (torch's scaled_dot_product_attention, float64);
  * closed forms: constant V gives gate*(1-lambda)*v, zero queries give a
    (windowed) prefix mean, a window of 1 gives gate*(1-lambda)*v_t;
  * invariants the equations fix: lambda = 1 with identical signal and noise
    queries gives exactly 0; a window >= T equals full causal; the output is
    affine in lambda with slope -gate*Repeat_4(H_N); batch independence;
    equivariance under a permutation of KV heads (with their groups);
  * brute force with an explicit masked score matrix and scipy's softmax;
  * decode equals the last prefill row.
Finally, each planted mistake in the oracle (ORACLE_MUTANT) must fail at
least one of these pins.
"""
import fractions
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from oracle import build as oracle_build

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_form_T3.txt")
D_QK, D_V, G = 192, 128, 4


def rand_inputs(B, T, n_kv, seed, q_std=0.3, k_std=0.3, v_std=1.0):
    """fp32 inputs with sharp-enough logits that every step of the softmax matters."""
    r = np.random.default_rng(seed)
    n_sig = n_kv * G
    return dict(
        q_signal=(r.standard_normal((B, T, n_sig, D_QK)) * q_std).astype(np.float32),
        q_noise=(r.standard_normal((B, T, n_kv, D_QK)) * q_std).astype(np.float32),
        k=(r.standard_normal((B, T, n_kv, D_QK)) * k_std).astype(np.float32),
        v=(r.standard_normal((B, T, n_kv, D_V)) * v_std).astype(np.float32),
        lam=r.uniform(0, 1, (B, T, n_sig)).astype(np.float32),
        gate=r.uniform(0, 1, (B, T, n_sig, D_V)).astype(np.float32),
    )


def run(x, window=0, scale=None, lib=None):
    return oracle.prefill(x["q_signal"], x["q_noise"], x["k"], x["v"], x["lam"], x["gate"],
                          window=window, scale=scale, lib=lib)


def band_mask(T, window):
    """Boolean [T,T] visibility: s <= t, and s > t-W with a window (torch.tril band)."""
    ones = torch.ones(T, T, dtype=torch.bool)
    m = torch.tril(ones)
    if window > 0:
        m = m & ~torch.tril(ones, diagonal=-window)
    return m


def sdpa_heads(q, k, v, window, scale):
    """Library attention per query head: q [B,T,H,d] against k/v [B,T,H,d] (float64)."""
    qt = torch.from_numpy(q).double().permute(0, 2, 1, 3)
    kt = torch.from_numpy(k).double().permute(0, 2, 1, 3)
    vt = torch.from_numpy(v).double().permute(0, 2, 1, 3)
    T = q.shape[1]
    o = torch.nn.functional.scaled_dot_product_attention(
        qt, kt, vt, attn_mask=band_mask(T, window), scale=scale)
    return o.permute(0, 2, 1, 3).numpy()


def kv_for_signal(a):
    """KV tensor [B,T,n_kv,d] expanded to the signal heads: head h reads KV head h//4."""
    return np.repeat(a, G, axis=2)


# ----------------------------------------------------------------------------
# 1. hand-derived closed form
# ----------------------------------------------------------------------------

def golden_inputs():
    T, n_kv = 3, 2
    n_sig = n_kv * G
    x = dict(q_signal=np.zeros((1, T, n_sig, D_QK), np.float32),
             q_noise=np.zeros((1, T, n_kv, D_QK), np.float32),
             k=np.zeros((1, T, n_kv, D_QK), np.float32),
             v=np.zeros((1, T, n_kv, D_V), np.float32),
             lam=np.zeros((1, T, n_sig), np.float32),
             gate=np.full((1, T, n_sig, D_V), 0.5, np.float32))
    for s in range(T):
        x["k"][0, s, 0, 0] = s
        x["k"][0, s, 1, 191] = 2 - s
        x["v"][0, s, 0, 0] = (1, 2, 3)[s]
        x["v"][0, s, 0, 1] = (4, 0, -4)[s]
        x["v"][0, s, 1, 0] = (2, 4, 8)[s]
        x["v"][0, s, 1, 127] = 1
    for t in range(T):
        for h, a in enumerate((1, 0, 2, -1)):
            x["q_signal"][0, t, h, 0] = a
        for h, a in enumerate((1, 2, 0, 1)):
            x["q_signal"][0, t, 4 + h, 191] = a
        x["q_noise"][0, t, 0, 0] = 1
        x["q_noise"][0, t, 1, 191] = -1
        for h in range(n_sig):
            x["lam"][0, t, h] = (h + 1) / 8
            x["gate"][0, t, h, 1] = 0.25
    return x


def golden_expected():
    rows = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            t, w, h, c, val = line.split()
            rows.append((int(t), int(w), int(h), int(c), float(fractions.Fraction(val))))
    return rows


def check_golden(lib=None):
    x = golden_inputs()
    exp = golden_expected()
    for window in (0, 2):
        out = run(x, window=window, scale=math.log(2.0), lib=lib)
        want = np.zeros_like(out)
        listed = np.zeros(out.shape, bool)
        for t, w, h, c, val in exp:
            if w == window:
                want[0, t, h, c] = val
                listed[0, t, h, c] = True
        # window 2 is only tabulated at t = 2 (rows 0, 1 are the full-causal rows)
        rows = slice(None) if window == 0 else slice(2, 3)
        np.testing.assert_allclose(out[:, rows], want[:, rows], rtol=0, atol=1e-12)
        assert listed.sum() > 0


def test_golden_closed_form():
    check_golden()


# ----------------------------------------------------------------------------
# 2. lambda = 0 reduces to library softmax attention on the signal heads
# ----------------------------------------------------------------------------

def check_lambda0_sdpa(lib=None, B=2, T=37, n_kv=3, windows=(0, 1, 5, 16)):
    x = rand_inputs(B, T, n_kv, seed=1)
    x["lam"][:] = 0
    scale = 1 / math.sqrt(D_QK)
    for window in windows:
        got = run(x, window=window, scale=scale, lib=lib)
        h = sdpa_heads(x["q_signal"], kv_for_signal(x["k"]), kv_for_signal(x["v"]), window, scale)
        np.testing.assert_allclose(got, x["gate"] * h, rtol=1e-11, atol=1e-12)


def test_lambda0_is_library_attention():
    check_lambda0_sdpa()


# ----------------------------------------------------------------------------
# 3. lambda = 1 with each group's signal queries equal to its noise query -> 0
# ----------------------------------------------------------------------------

def check_lambda1_zero(lib=None, B=1, T=29, n_kv=3, window=0):
    x = rand_inputs(B, T, n_kv, seed=2)
    x["q_signal"] = np.repeat(x["q_noise"], G, axis=2).copy()   # signal 4j..4j+3 <- noise j
    x["lam"][:] = 1
    out = run(x, window=window, lib=lib)
    assert np.max(np.abs(out)) == 0.0


def test_lambda1_identical_queries_give_zero():
    for window in (0, 7):
        check_lambda1_zero(window=window)


# ----------------------------------------------------------------------------
# 4. window >= T equals full causal (bitwise in the oracle)
# ----------------------------------------------------------------------------

def test_window_at_least_T_is_full_causal():
    x = rand_inputs(1, 23, 2, seed=3)
    full = run(x, window=0)
    for window in (23, 24, 1000):
        assert np.array_equal(run(x, window=window), full)


# ----------------------------------------------------------------------------
# 5. closed forms: constant V, zero queries, window 1
# ----------------------------------------------------------------------------

def check_constant_v(lib=None, window=0):
    B, T, n_kv = 2, 19, 3
    x = rand_inputs(B, T, n_kv, seed=4)
    c = np.random.default_rng(5).standard_normal((n_kv, D_V)).astype(np.float32)
    x["v"][:] = c[None, None]
    out = run(x, window=window, lib=lib)
    want = x["gate"].astype(np.float64) * (1 - x["lam"].astype(np.float64))[..., None] \
        * np.repeat(c, G, axis=0).astype(np.float64)[None, None]
    np.testing.assert_allclose(out, want, rtol=1e-12, atol=1e-13)


def test_constant_v_gives_gate_times_one_minus_lambda_times_v():
    for window in (0, 4):
        check_constant_v(window=window)


def check_zero_q_prefix_mean(lib=None, windows=(0, 1, 5, 12)):
    B, T, n_kv = 2, 31, 2
    x = rand_inputs(B, T, n_kv, seed=6)
    x["q_signal"][:] = 0
    x["q_noise"][:] = 0
    v = x["v"].astype(np.float64)
    csum = np.concatenate([np.zeros((B, 1, n_kv, D_V)), np.cumsum(v, axis=1)], axis=1)
    for window in windows:
        t = np.arange(T)
        lo = np.maximum(0, t - window + 1) if window > 0 else np.zeros(T, int)
        mean = (csum[:, t + 1] - csum[:, lo]) / (t + 1 - lo)[None, :, None, None]
        want = x["gate"] * (1 - x["lam"].astype(np.float64))[..., None] * np.repeat(mean, G, axis=2)
        np.testing.assert_allclose(run(x, window=window, lib=lib), want, rtol=1e-11, atol=1e-12)


def test_zero_queries_give_windowed_prefix_mean():
    check_zero_q_prefix_mean()


def test_window_one_and_first_row_see_only_themselves():
    x = rand_inputs(2, 17, 2, seed=7)
    own = x["gate"] * (1 - x["lam"].astype(np.float64))[..., None] * np.repeat(x["v"], G, axis=2)
    np.testing.assert_allclose(run(x, window=1), own, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(run(x, window=0)[:, 0], own[:, 0], rtol=1e-12, atol=1e-13)


# ----------------------------------------------------------------------------
# 6. affine in lambda: slope is -gate * Repeat_4(H_N), H_N from library attention
# ----------------------------------------------------------------------------

def check_affine_lambda(lib=None, window=0):
    B, T, n_kv = 1, 27, 3
    x = rand_inputs(B, T, n_kv, seed=8)
    x2 = dict(x)
    x2["lam"] = np.random.default_rng(9).uniform(0, 1, x["lam"].shape).astype(np.float32)
    scale = 1 / math.sqrt(D_QK)
    diff = run(x, window, scale, lib) - run(x2, window, scale, lib)
    hn = sdpa_heads(x["q_noise"], x["k"], x["v"], window, scale)          # [B,T,n_kv,D_V]
    want = -(x["lam"].astype(np.float64) - x2["lam"])[..., None] * x["gate"] \
        * np.repeat(hn, G, axis=2)
    np.testing.assert_allclose(diff, want, rtol=1e-9, atol=1e-12)


def test_affine_in_lambda_with_noise_path_slope():
    for window in (0, 6):
        check_affine_lambda(window=window)


# ----------------------------------------------------------------------------
# 7. brute force: explicit masked [T,T] scores, scipy softmax
# ----------------------------------------------------------------------------

def brute_force(x, window, scale):
    q_s, q_n = x["q_signal"].astype(np.float64), x["q_noise"].astype(np.float64)
    k, v = x["k"].astype(np.float64), x["v"].astype(np.float64)
    B, T, n_kv, _ = k.shape
    vis = band_mask(T, window).numpy()
    out = np.zeros((B, T, n_kv * G, D_V))
    for b in range(B):
        for j in range(n_kv):
            def attn(q):
                s = scale * q @ k[b, :, j].T
                s[~vis] = -np.inf
                return scipy.special.softmax(s, axis=1) @ v[b, :, j]
            hn = attn(q_n[b, :, j])
            for i in range(G):
                h = G * j + i
                d = attn(q_s[b, :, h]) - x["lam"][b, :, h, None] * hn
                out[b, :, h] = x["gate"][b, :, h] * d
    return out


@pytest.mark.parametrize("T,window,B,n_kv", [
    (1, 0, 1, 1), (2, 0, 2, 1), (3, 1, 1, 2), (5, 2, 1, 3), (64, 0, 1, 1), (127, 128, 1, 1),
    (128, 127, 1, 1), (129, 128, 2, 1), (129, 129, 1, 2), (200, 0, 1, 1)])
def test_brute_force_explicit_scores(T, window, B, n_kv):
    x = rand_inputs(B, T, n_kv, seed=T * 7 + window)
    scale = 1 / math.sqrt(D_QK)
    np.testing.assert_allclose(run(x, window, scale), brute_force(x, window, scale),
                               rtol=1e-10, atol=1e-12)


# ----------------------------------------------------------------------------
# 8. independence and equivariance
# ----------------------------------------------------------------------------

def test_batch_independence():
    x = rand_inputs(2, 21, 2, seed=10)
    a = run(x, window=0)
    y = {k: v.copy() for k, v in x.items()}
    for key in y:
        y[key][1] = rand_inputs(1, 21, 2, seed=11)[key][0]
    b = run(y, window=0)
    assert np.array_equal(a[0], b[0])
    assert not np.allclose(a[1], b[1])


def test_kv_head_permutation_equivariance():
    x = rand_inputs(1, 15, 3, seed=12)
    perm = np.array([2, 0, 1])
    sig_perm = (perm[:, None] * G + np.arange(G)[None]).reshape(-1)
    y = dict(q_signal=x["q_signal"][:, :, sig_perm], q_noise=x["q_noise"][:, :, perm],
             k=x["k"][:, :, perm], v=x["v"][:, :, perm], lam=x["lam"][:, :, sig_perm],
             gate=x["gate"][:, :, sig_perm])
    y = {k: np.ascontiguousarray(v) for k, v in y.items()}
    for window in (0, 5):
        assert np.array_equal(run(y, window)[:, :, :], run(x, window)[:, :, sig_perm])


# ----------------------------------------------------------------------------
# 9. decode equals the last prefill row; sampled rows equal full rows
# ----------------------------------------------------------------------------

def pack_decode(seqs):
    """Pack per-sequence prefill inputs into decode inputs (query = last position)."""
    lengths = [s["k"].shape[1] for s in seqs]
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    return dict(
        q_signal=np.stack([s["q_signal"][0, -1] for s in seqs]),
        q_noise=np.stack([s["q_noise"][0, -1] for s in seqs]),
        k_cache=np.concatenate([s["k"][0] for s in seqs]),
        v_cache=np.concatenate([s["v"][0] for s in seqs]),
        cu_seqlens=cu,
        lam=np.stack([s["lam"][0, -1] for s in seqs]),
        gate=np.stack([s["gate"][0, -1] for s in seqs])), lengths


def test_decode_equals_last_prefill_row():
    seqs = [rand_inputs(1, L, 2, seed=20 + L) for L in (1, 2, 9, 40, 131)]
    d, lengths = pack_decode(seqs)
    for window in (0, 1, 8, 128):
        got = oracle.decode(d["q_signal"], d["q_noise"], d["k_cache"], d["v_cache"],
                            d["cu_seqlens"], d["lam"], d["gate"], window=window)
        for b, s in enumerate(seqs):
            want = run(s, window=window)[0, -1]
            assert np.array_equal(got[b], want)


def test_sampled_rows_equal_full_rows():
    x = rand_inputs(2, 33, 2, seed=30)
    full = run(x, window=9)
    rb = np.array([0, 1, 1, 0], np.int32)
    rt = np.array([0, 32, 5, 17], np.int32)
    rows = oracle.prefill_rows(x["k"], x["v"], x["q_signal"][rb, rt], x["q_noise"][rb, rt],
                               x["lam"][rb, rt], x["gate"][rb, rt], rb, rt, window=9)
    assert np.array_equal(rows, full[rb, rt])


def test_oracle_rejects_bad_arguments():
    x = rand_inputs(1, 4, 1, seed=31)
    with pytest.raises(ValueError):
        oracle.prefill_rows(x["k"], x["v"], x["q_signal"][0], x["q_noise"][0], x["lam"][0],
                            x["gate"][0], [0, 0, 0, 0], [0, 1, 2, 4])     # t out of range
    with pytest.raises(ValueError):
        oracle.decode(x["q_signal"][:, 0], x["q_noise"][:, 0], x["k"][0], x["v"][0],
                      np.array([0, 0], np.int32), x["lam"][:, 0], x["gate"][:, 0])   # empty


# ----------------------------------------------------------------------------
# 10. latent-cache decode: the same result as the expanded cache it stands for
# ----------------------------------------------------------------------------

def latent_inputs(lengths, n_kv, seed, d_c=512, d_r=64, d_kc=128, d_v=128):
    r = np.random.default_rng(seed)
    B, n_sig = len(lengths), 4 * n_kv
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    total = int(cu[-1])
    f = lambda *shape, s=1.0: (r.standard_normal(shape) * s).astype(np.float32)
    return dict(q_signal=f(B, n_sig, d_kc + d_r, s=0.3), q_noise=f(B, n_kv, d_kc + d_r, s=0.3),
                latent=f(total, d_c + d_r), w_uk=f(n_kv, d_kc, d_c, s=0.05),
                w_uv=f(n_kv, d_v, d_c, s=0.05), cu_seqlens=cu,
                lam=r.uniform(0, 1, (B, n_sig)).astype(np.float32),
                gate=r.uniform(0, 1, (B, n_sig, d_v)).astype(np.float32))


def expand_latent(x, d_c=512):
    """Per-head K and V by explicit up-projection (numpy, float64)."""
    c = x["latent"][:, :d_c].astype(np.float64)
    kr = x["latent"][:, d_c:].astype(np.float64)
    kc = np.einsum("jdc,sc->sjd", x["w_uk"].astype(np.float64), c)
    k = np.concatenate([kc, np.broadcast_to(kr[:, None, :], (c.shape[0], kc.shape[1], kr.shape[1]))],
                       axis=2)
    v = np.einsum("jdc,sc->sjd", x["w_uv"].astype(np.float64), c)
    return k, v


def latent_oracle(x, window, lib=None):
    return oracle.decode_latent(x["q_signal"], x["q_noise"], x["latent"], x["w_uk"], x["w_uv"],
                                x["cu_seqlens"], x["lam"], x["gate"], window=window, lib=lib)


def check_latent_equals_expanded(lib=None, windows=(0, 1, 5)):
    x = latent_inputs([1, 7, 23], 2, seed=40)
    k, v = expand_latent(x)
    for window in windows:
        got = latent_oracle(x, window, lib)
        # the expanded path is pinned above; K and V widen from float64 to its float32 inputs
        want = oracle.decode(x["q_signal"], x["q_noise"], k.astype(np.float32), v.astype(np.float32),
                             x["cu_seqlens"], x["lam"], x["gate"], window=window)
        np.testing.assert_allclose(got, want, rtol=1e-5, atol=1e-6)


def test_latent_decode_equals_expanded_decode():
    check_latent_equals_expanded()


def check_latent_window_one(lib=None):
    # W = 1: each sequence's query sees only its last row, so out = gate (1 - lambda) W_uv[j] c_last
    x = latent_inputs([3, 1, 12], 3, seed=41)
    got = latent_oracle(x, 1, lib)
    last = x["latent"][x["cu_seqlens"][1:] - 1, :512].astype(np.float64)        # [B, 512]
    vj = np.einsum("jdc,bc->bjd", x["w_uv"].astype(np.float64), last)           # [B, n_kv, 128]
    want = (x["gate"].astype(np.float64) * (1.0 - x["lam"].astype(np.float64))[:, :, None]
            * np.repeat(vj, 4, axis=1))
    np.testing.assert_allclose(got, want, rtol=1e-9, atol=1e-12)


def test_latent_window_one_is_last_value():
    check_latent_window_one()


def test_latent_lambda1_identical_queries_give_zero():
    x = latent_inputs([5, 30], 2, seed=42)
    x["q_signal"] = np.repeat(x["q_noise"], 4, axis=1)
    x["lam"] = np.ones_like(x["lam"])
    assert np.array_equal(latent_oracle(x, 0), np.zeros_like(x["gate"], dtype=np.float64))


# ----------------------------------------------------------------------------
# 10b. the step ahead of the attention core: rotary embedding, lambda, gate
# ----------------------------------------------------------------------------

def prep_inputs(B=1, T=3, n_kv=2, d_model=64, seed=0):
    r = np.random.default_rng(seed)
    f = lambda *s: r.standard_normal(s).astype(np.float32)
    n_sig = 4 * n_kv
    return dict(q_signal=f(B, T, n_sig, 192), q_noise=f(B, T, n_kv, 192), k_rope=f(B, T, 64),
                x=f(B, T, d_model), w_lambda=(0.1 * f(n_sig, d_model)).astype(np.float32),
                gate_pre=f(B, T, n_sig, 128))


def run_prep(lib, d, **kw):
    return oracle.prep(d["q_signal"], d["q_noise"], d["k_rope"], d["x"], d["w_lambda"], d["gate_pre"],
                       lib=lib, **kw)


def check_rope_closed_form(lib):
    """Unit vectors turn by a known angle in a known plane: e_0 at position 1 by
    1 radian in the plane of values 0, 1 (pair 0 turns at theta^0 = 1 per
    position); e_32 at position 100 by 100 * 10000^(-32/64) = 1 radian in the
    plane of values 32, 33 (pair 16).  Query heads carry the rotary part in
    their last 64 values; every KV head receives the rotated shared key."""
    d = prep_inputs(T=1)
    for pos0, unit, plane in [(1, 0, (0, 1)), (100, 32, (32, 33))]:
        e = dict(d)
        e["q_signal"] = np.zeros_like(d["q_signal"])
        e["q_signal"][..., 128 + unit] = 1.0
        e["k_rope"] = np.zeros_like(d["k_rope"])
        e["k_rope"][..., unit] = 1.0
        o = run_prep(lib, e, pos0=pos0, theta=10000.0)
        want = np.zeros(64)
        want[plane[0]], want[plane[1]] = math.cos(1.0), math.sin(1.0)
        np.testing.assert_allclose(o["q_signal"][0, 0, :, 128:], np.broadcast_to(want, (8, 64)), atol=1e-12)
        np.testing.assert_allclose(o["k_rot"][0, 0], np.broadcast_to(want, (2, 64)), atol=1e-12)


def check_rope_relative_norm_identity(lib):
    """The defining property of the rotary embedding: the dot product of a
    rotated query and a rotated key depends on their positions only through
    the difference; every pair keeps its length; position 0 is the identity."""
    d = prep_inputs(T=5, n_kv=1)
    a = run_prep(lib, d, pos0=0, theta=10000.0)
    b = run_prep(lib, d, pos0=37, theta=10000.0)
    sa = np.einsum("thd,sd->ths", a["q_signal"][0, :, :, 128:], a["k_rot"][0, :, 0])
    sb = np.einsum("thd,sd->ths", b["q_signal"][0, :, :, 128:], b["k_rot"][0, :, 0])
    np.testing.assert_allclose(sa, sb, rtol=1e-9, atol=1e-9)
    pairs = lambda v: np.linalg.norm(v.reshape(*v.shape[:-1], 32, 2), axis=-1)
    np.testing.assert_allclose(pairs(b["q_noise"][..., 128:]), pairs(d["q_noise"][..., 128:].astype(np.float64)),
                               rtol=1e-12)
    np.testing.assert_allclose(a["q_signal"][0, 0], d["q_signal"][0, 0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(a["k_rot"][0, 0, 0], d["k_rope"][0, 0], rtol=0, atol=1e-12)


def check_prep_structure(lib):
    """The content part (first 128 values) of every query head passes unchanged,
    and every KV head receives the same rotated key."""
    d = prep_inputs(T=4, n_kv=3)
    o = run_prep(lib, d, pos0=9, theta=10000.0)
    np.testing.assert_array_equal(o["q_signal"][..., :128], d["q_signal"][..., :128])
    np.testing.assert_array_equal(o["q_noise"][..., :128], d["q_noise"][..., :128])
    for j in range(1, 3):
        np.testing.assert_array_equal(o["k_rot"][:, :, j], o["k_rot"][:, :, 0])


def check_lambda_gate_sigmoid(lib):
    """lambda = sigmoid(x . W^lambda[h]) and gate = sigmoid(pre-activation):
    zero weights or pre-activations give exactly 1/2; negating the input gives
    1 - value; a one-hot x picks out a single weight."""
    d = prep_inputs(T=2)
    o = run_prep(lib, d, pos0=0, theta=10000.0)
    z = dict(d, w_lambda=np.zeros_like(d["w_lambda"]), gate_pre=np.zeros_like(d["gate_pre"]))
    oz = run_prep(lib, z)
    assert np.all(oz["lam"] == 0.5) and np.all(oz["gate"] == 0.5)
    neg = run_prep(lib, dict(d, x=-d["x"], gate_pre=-d["gate_pre"]))
    np.testing.assert_allclose(neg["lam"], 1.0 - o["lam"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(neg["gate"], 1.0 - o["gate"], rtol=0, atol=1e-14)
    onehot = np.zeros_like(d["x"])
    onehot[..., 5] = 1.0
    oh = run_prep(lib, dict(d, x=onehot))
    w5 = d["w_lambda"][:, 5].astype(np.float64)
    np.testing.assert_allclose(oh["lam"][0, 0], 1.0 / (1.0 + np.exp(-w5)), rtol=1e-14)
    assert np.all((o["lam"] > 0) & (o["lam"] < 1))


def test_rope_closed_form():
    check_rope_closed_form(oracle.library())


def test_rope_relative_position_norm_identity():
    check_rope_relative_norm_identity(oracle.library())


def test_prep_structure():
    check_prep_structure(oracle.library())


def test_lambda_and_gate_are_sigmoids():
    check_lambda_gate_sigmoid(oracle.library())


def test_prep_rejects_bad_arguments():
    d = prep_inputs()
    with pytest.raises(ValueError):
        run_prep(oracle.library(), d, pos0=-1)
    with pytest.raises(ValueError):
        run_prep(oracle.library(), d, theta=1.0)


# ----------------------------------------------------------------------------
# 11. every planted mistake fails at least one pin
# ----------------------------------------------------------------------------

MUTANTS = {
    1: "Repeat_4 tiled instead of interleaved",
    2: "wrong sign in the differential combine",
    3: "window one key too wide",
    4: "gate not applied",
    5: "rotary tail of the query-key dot product dropped",
    6: "softmax scale forgotten",
    7: "V read from the wrong KV head",
    8: "latent decode: rotary key dropped",
    9: "latent decode: W_uk read transposed",
    10: "latent decode: values up-projected with W_uk",
    11: "rotary pairs taken as halves (i, i+32) instead of adjacent values",
    12: "rotation turned the wrong way",
    13: "rotary frequencies theta^(-i/64) instead of theta^(-2i/64)",
    14: "lambda and gate without the sigmoid",
    15: "shared rotary key left unrotated in KV heads past the first",
    16: "rotary embedding applied to the first 64 values of a head",
}


def pin_suite(lib):
    """The pins above, pointed at a given oracle build; returns the names that fail."""
    checks = {
        "golden": lambda: check_golden(lib),
        "lambda0_sdpa": lambda: check_lambda0_sdpa(lib, B=1, T=17, n_kv=3, windows=(0, 5)),
        "lambda1_zero": lambda: check_lambda1_zero(lib, T=9),
        "constant_v": lambda: check_constant_v(lib),
        "zero_q_mean": lambda: check_zero_q_prefix_mean(lib, windows=(0, 5)),
        "affine_lambda": lambda: check_affine_lambda(lib),
        "latent_expanded": lambda: check_latent_equals_expanded(lib, windows=(0, 5)),
        "latent_window_one": lambda: check_latent_window_one(lib),
        "rope_closed_form": lambda: check_rope_closed_form(lib),
        "rope_relative": lambda: check_rope_relative_norm_identity(lib),
        "prep_structure": lambda: check_prep_structure(lib),
        "lambda_gate_sigmoid": lambda: check_lambda_gate_sigmoid(lib),
    }
    failed = []
    for name, fn in checks.items():
        try:
            fn()
        except AssertionError:
            failed.append(name)
    return failed


def test_unmutated_oracle_passes_pin_suite():
    assert pin_suite(oracle.library()) == []


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_planted_mistake_is_caught(mutant, tmp_path):
    path = oracle_build.build_oracle(out_dir=str(tmp_path), mutant=mutant)
    failed = pin_suite(oracle.library(path))
    assert failed, "planted mistake %d (%s) passed every pin" % (mutant, MUTANTS[mutant])
