"""Pins of the gradient oracle (oracle/backward.py), CPU only.

The oracle's forward is checked against the C oracle (an independent
implementation of the same definition), its gradients against central finite
differences of that forward, and both against identities of the softmax.  A
planted mistake in the forward must fail the first pin.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import backward as ob


def inputs(B=1, T=9, n_kv=2, seed=0, q_std=1.0):
    g = torch.Generator().manual_seed(seed)
    r = lambda *s, std=1.0: torch.randn(s, generator=g, dtype=torch.float64) * std
    n_sig = 4 * n_kv
    return dict(q_signal=r(B, T, n_sig, 192, std=q_std), q_noise=r(B, T, n_kv, 192, std=q_std),
                k=r(B, T, n_kv, 192, std=1 / math.sqrt(192) * 4), v=r(B, T, n_kv, 128),
                lam=torch.rand(B, T, n_sig, generator=g, dtype=torch.float64),
                gate=torch.sigmoid(r(B, T, n_sig, 128)))


def c_oracle(x, window):
    f = lambda t: t.float().numpy()
    return oracle.prefill(f(x["q_signal"]), f(x["q_noise"]), f(x["k"]), f(x["v"]), f(x["lam"]), f(x["gate"]),
                          window=window)


def as_f32(x):
    """Inputs rounded to float32 (the C oracle reads float32), kept in float64."""
    return {k: v.float().double() for k, v in x.items()}


@pytest.mark.parametrize("window", [0, 1, 4, 100])
def test_forward_equals_c_oracle(window):
    x = as_f32(inputs(B=2, T=11, n_kv=2, seed=1))
    got = ob.forward(*[x[n] for n in ob.NAMES], window=window).numpy()
    np.testing.assert_allclose(got, c_oracle(x, window), rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("mutant", [1, 2, 3])
def test_planted_forward_mistake_is_caught(mutant):
    """1: Repeat_g tiled instead of interleaved; 2: window one key too wide;
    3: softmax scale forgotten."""
    x = as_f32(inputs(B=1, T=9, n_kv=2, seed=2))
    got = ob.forward(*[x[n] for n in ob.NAMES], window=4, mutant=mutant).numpy()
    assert not np.allclose(got, c_oracle(x, 4), rtol=1e-6, atol=1e-8)


@pytest.mark.parametrize("window", [0, 3])
def test_gradients_equal_finite_differences(window):
    """<grad_x, u> equals (L(x + eps u) - L(x - eps u)) / (2 eps) for
    L = sum(d_out * out) and a random direction u, for each input x."""
    x = inputs(B=1, T=6, n_kv=1, seed=3)
    d_out = torch.randn(1, 6, 4, 128, generator=torch.Generator().manual_seed(4), dtype=torch.float64)
    grads = ob.backward(*[x[n] for n in ob.NAMES], d_out, window=window)
    gen = torch.Generator().manual_seed(5)
    eps = 1e-5
    for name in ob.NAMES:
        u = torch.randn(x[name].shape, generator=gen, dtype=torch.float64)
        def loss(delta):
            y = dict(x)
            y[name] = x[name] + delta * u
            return float((ob.forward(*[y[n] for n in ob.NAMES], window=window) * d_out).sum())
        fd = (loss(eps) - loss(-eps)) / (2 * eps)
        an = float((grads[name] * u).sum())
        assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (name, fd, an)


def test_softmax_identities():
    """Every query row's softmax weights sum to one, so the key gradients of a
    KV head sum to zero over the keys, and its value gradients sum to the
    output gradients of its five heads: gate (.) d_out for the signal heads and
    -sum_h lambda_h gate_h (.) d_out_h for the noise head."""
    x = inputs(B=2, T=10, n_kv=2, seed=6)
    d_out = torch.randn(2, 10, 8, 128, generator=torch.Generator().manual_seed(7), dtype=torch.float64)
    for window in (0, 3):
        gr = ob.backward(*[x[n] for n in ob.NAMES], d_out, window=window)
        np.testing.assert_allclose(gr["k"].sum(dim=1).numpy(), 0.0, atol=1e-10)
        dd = x["gate"] * d_out                                           # d out / d D
        dhn = -(x["lam"][..., None] * dd).reshape(2, 10, 2, 4, 128).sum(dim=3)
        want = dd.reshape(2, 10, 2, 4, 128).sum(dim=3) + dhn             # per KV head
        np.testing.assert_allclose(gr["v"].sum(dim=1).numpy(), want.sum(dim=1).numpy(), rtol=1e-10, atol=1e-10)


def test_gate_zero_and_lambda_zero():
    """gate = 0 removes every path but the gate's own: its gradient is
    d_out (.) D; lambda = 0 removes the noise path."""
    x = inputs(B=1, T=7, n_kv=2, seed=8)
    d_out = torch.randn(1, 7, 8, 128, generator=torch.Generator().manual_seed(9), dtype=torch.float64)
    z = dict(x, gate=torch.zeros_like(x["gate"]))
    gr = ob.backward(*[z[n] for n in ob.NAMES], d_out)
    for n in ("q_signal", "q_noise", "k", "v", "lam"):
        assert float(gr[n].abs().max()) == 0.0, n
    _, hs, hn = ob.forward(*[x[n] for n in ob.NAMES], parts=True)
    dmat = hs - x["lam"][..., None] * hn.repeat_interleave(4, dim=2)
    np.testing.assert_allclose(gr["gate"].numpy(), (d_out * dmat).numpy(), rtol=1e-12, atol=1e-14)
    z = dict(x, lam=torch.zeros_like(x["lam"]))
    gr = ob.backward(*[z[n] for n in ob.NAMES], d_out)
    assert float(gr["q_noise"].abs().max()) == 0.0


def test_gradients_match_c_oracle_differences():
    """The same directional check against the C oracle's forward, which shares
    nothing with the torch one.  The C oracle reads float32, so the perturbed
    points are float32 and the step actually taken, x+ - x-, is the direction."""
    x = as_f32(inputs(B=1, T=7, n_kv=1, seed=10))
    d_out = torch.randn(1, 7, 4, 128, generator=torch.Generator().manual_seed(11), dtype=torch.float64)
    grads = ob.backward(*[x[n] for n in ob.NAMES], d_out, window=3)
    gen = torch.Generator().manual_seed(12)
    for name in ob.NAMES:
        u = torch.randn(x[name].shape, generator=gen, dtype=torch.float64) * 3e-3 * float(x[name].abs().mean())
        xp, xm = dict(x), dict(x)
        xp[name] = (x[name] + u).float().double()
        xm[name] = (x[name] - u).float().double()
        step = xp[name] - xm[name]
        fd = float((torch.from_numpy(c_oracle(xp, 3) - c_oracle(xm, 3)) * d_out).sum())
        an = float((grads[name] * step).sum())
        assert abs(fd - an) <= 1e-3 * abs(an) + 1e-9, (name, fd, an)
