"""Pins for the float64 torch row oracle (oracle/rows.py), which checks the
longest workloads on sampled rows.

It is pinned independently of its own code: it must equal the C oracle (itself
pinned by tests/test_oracle_pins.py) on random inputs, reproduce the
hand-derived closed form of tests/golden/closed_form_T3.txt, reduce to torch's
scaled_dot_product_attention at lambda = 0, match the explicit-score brute
force, and give the same rows whatever chunks it splits them into.  Each of
its planted mistakes must fail one of these.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import rows as orows
from test_oracle_pins import (D_QK, G, brute_force, golden_expected, golden_inputs, kv_for_signal, rand_inputs,
                              sdpa_heads)


def run_rows(x, window=0, scale=None, rb=None, rt=None, mutant=0):
    B, T = x["k"].shape[:2]
    if rb is None:
        bb, tt = np.meshgrid(np.arange(B), np.arange(T), indexing="ij")
        rb, rt = bb.reshape(-1), tt.reshape(-1)
    pick = lambda a: torch.from_numpy(np.ascontiguousarray(a[rb, rt]))
    out = orows.prefill_rows(torch.from_numpy(x["k"]), torch.from_numpy(x["v"]), pick(x["q_signal"]),
                             pick(x["q_noise"]), pick(x["lam"]), pick(x["gate"]), rb, rt, window=window,
                             scale=scale, mutant=mutant).numpy()
    return out


def full_shape(x, out):
    B, T = x["k"].shape[:2]
    return out.reshape(B, T, *out.shape[1:])


def check_equals_c_oracle(mutant=0):
    x = rand_inputs(2, 150, 3, seed=31)
    r = np.random.default_rng(32)
    rb = np.concatenate([[0, 1, 1, 0], r.integers(0, 2, 40)]).astype(np.int32)
    rt = np.concatenate([[0, 149, 0, 149], r.integers(0, 150, 40)]).astype(np.int32)
    for window in (0, 1, 5, 40):
        want = oracle.prefill_rows(x["k"], x["v"], x["q_signal"][rb, rt], x["q_noise"][rb, rt], x["lam"][rb, rt],
                                   x["gate"][rb, rt], rb, rt, window=window)
        got = run_rows(x, window, rb=rb, rt=rt, mutant=mutant)
        np.testing.assert_allclose(got, want, rtol=1e-10, atol=1e-12)


def test_rows_equal_c_oracle():
    check_equals_c_oracle()


def check_golden(mutant=0):
    x = golden_inputs()
    for window in (0, 2):
        out = full_shape(x, run_rows(x, window, scale=math.log(2.0), mutant=mutant))
        want = np.zeros_like(out)
        for t, w, h, c, val in golden_expected():
            if w == window:
                want[0, t, h, c] = val
        rows = slice(None) if window == 0 else slice(2, 3)
        np.testing.assert_allclose(out[:, rows], want[:, rows], rtol=0, atol=1e-12)


def test_rows_golden_closed_form():
    check_golden()


def check_lambda0_sdpa(mutant=0):
    x = rand_inputs(2, 37, 3, seed=1)
    x["lam"][:] = 0
    scale = 1 / math.sqrt(D_QK)
    for window in (0, 1, 5, 16):
        got = full_shape(x, run_rows(x, window, scale, mutant=mutant))
        h = sdpa_heads(x["q_signal"], kv_for_signal(x["k"]), kv_for_signal(x["v"]), window, scale)
        np.testing.assert_allclose(got, x["gate"] * h, rtol=1e-11, atol=1e-12)


def test_rows_lambda0_is_library_attention():
    check_lambda0_sdpa()


def check_brute_force(mutant=0):
    for T, window in ((1, 0), (5, 2), (70, 0), (129, 128), (100, 7)):
        x = rand_inputs(1, T, 2, seed=T + window)
        scale = 1 / math.sqrt(D_QK)
        np.testing.assert_allclose(full_shape(x, run_rows(x, window, scale, mutant=mutant)),
                                   brute_force(x, window, scale), rtol=1e-10, atol=1e-12)


def test_rows_brute_force():
    check_brute_force()


def test_rows_independent_of_chunking(monkeypatch):
    """Long rows split into many small chunks give the same rows (to the last
    few bits: the library's matmul may block differently)."""
    x = rand_inputs(1, 3000, 2, seed=33)
    r = np.random.default_rng(34)
    rt = np.unique(np.concatenate([[0, 1, 2999], r.integers(0, 3000, 60)])).astype(np.int32)
    rb = np.zeros_like(rt)
    for window in (0, 128):
        one = run_rows(x, window, rb=rb, rt=rt)
        monkeypatch.setattr(orows, "_CHUNK_ELEMS", 40_000)
        many = run_rows(x, window, rb=rb, rt=rt)
        monkeypatch.undo()
        np.testing.assert_allclose(many, one, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("mutant", [1, 2, 3, 4])
def test_rows_planted_mistakes_are_caught(mutant):
    checks = (check_equals_c_oracle, check_golden, check_lambda0_sdpa, check_brute_force)
    failed = 0
    for chk in checks:
        try:
            chk(mutant)
        except AssertionError:
            failed += 1
    assert failed >= 1, "planted mistake %d passed every pin" % mutant
