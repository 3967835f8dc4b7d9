"""Pins for the fp32 build of the C oracle (the same source with its prefill
and decode definitions carried in fp32), the CPU reference whose speed the
benchmark reports.  The same pins as the fp64 build, at fp32 tolerances: the
hand-derived closed form, library attention at lambda = 0, the brute force,
exact zero at lambda = 1 with identical queries, window >= T, and agreement
with the fp64 build."""
import math

import numpy as np
import pytest

import oracle
from test_oracle_pins import (D_QK, brute_force, golden_expected, golden_inputs, kv_for_signal, pack_decode,
                              rand_inputs, run, sdpa_heads)


@pytest.fixture(scope="module")
def lib32():
    return oracle.library_fp32()


def test_fp32_golden_closed_form(lib32):
    x = golden_inputs()
    for window in (0, 2):
        out = run(x, window=window, scale=math.log(2.0), lib=lib32)
        want = np.zeros_like(out)
        for t, w, h, c, val in golden_expected():
            if w == window:
                want[0, t, h, c] = val
        rows = slice(None) if window == 0 else slice(2, 3)
        np.testing.assert_allclose(out[:, rows], want[:, rows], rtol=0, atol=4e-6)


def test_fp32_lambda0_is_library_attention(lib32):
    x = rand_inputs(2, 37, 3, seed=1)
    x["lam"][:] = 0
    scale = 1 / math.sqrt(D_QK)
    for window in (0, 1, 5, 16):
        got = run(x, window=window, scale=scale, lib=lib32)
        h = sdpa_heads(x["q_signal"], kv_for_signal(x["k"]), kv_for_signal(x["v"]), window, scale)
        np.testing.assert_allclose(got, x["gate"] * h, rtol=2e-5, atol=2e-6)


@pytest.mark.parametrize("T,window", [(1, 0), (5, 2), (64, 0), (129, 128), (200, 7)])
def test_fp32_brute_force(lib32, T, window):
    x = rand_inputs(1, T, 2, seed=T * 7 + window)
    scale = 1 / math.sqrt(D_QK)
    np.testing.assert_allclose(run(x, window, scale, lib32), brute_force(x, window, scale), rtol=2e-5, atol=2e-6)


def test_fp32_lambda1_zero_and_window_ge_T(lib32):
    x = rand_inputs(1, 29, 3, seed=2)
    x["q_signal"] = np.repeat(x["q_noise"], 4, axis=2).copy()
    x["lam"][:] = 1
    assert np.max(np.abs(run(x, window=0, lib=lib32))) == 0.0
    y = rand_inputs(1, 23, 2, seed=3)
    assert np.array_equal(run(y, window=23, lib=lib32), run(y, window=0, lib=lib32))


def test_fp32_close_to_fp64(lib32):
    x = rand_inputs(2, 300, 2, seed=40)
    for window in (0, 128):
        a = run(x, window=window, lib=lib32)
        b = run(x, window=window)
        assert np.linalg.norm(a - b) / np.linalg.norm(b) < 1e-5
    seqs = [rand_inputs(1, L, 2, seed=41 + L) for L in (1, 70, 300)]
    d, _ = pack_decode(seqs)
    args = (d["q_signal"], d["q_noise"], d["k_cache"], d["v_cache"], d["cu_seqlens"], d["lam"], d["gate"])
    a = oracle.decode(*args, lib=lib32)
    b = oracle.decode(*args)
    assert np.linalg.norm(a - b) / np.linalg.norm(b) < 1e-5
