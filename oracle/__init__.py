"""CPU oracle for the GDLA attention core -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product library under
``attention_gdla_prefill_amd`` never imports it, and the two share no code.

The arithmetic lives in ``gdla_oracle.c`` (plain C, fp64 sums and exponentials,
two-pass softmax; :func:`library_fp32` loads the same source built with fp32
arithmetic).  This module only marshals numpy arrays into it:

* :func:`prefill` -- every query position of a [B, T] prefill;
* :func:`prefill_rows` -- a chosen list of (b, t) positions, for workloads too
  large to check in full (the oracle is per row, so sampling is exact);
* :func:`decode` -- one new query per sequence over a packed KV cache;
* :func:`decode_latent` -- the same over a latent (compressed) KV cache, with
  the per-head keys and values formed by explicit up-projection;
* :func:`prep` -- the step ahead of the attention core: rotary embedding of
  the query heads and of the shared rotary key, lambda and the gate.

Inputs are float32 arrays (bf16 tensors widen to float32 exactly); outputs are
float64 arrays, never rounded.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_LIB = None

_f32p = np.ctypeslib.ndpointer(dtype=np.float32, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(dtype=np.float64, flags="C_CONTIGUOUS")
_i32p = np.ctypeslib.ndpointer(dtype=np.int32, flags="C_CONTIGUOUS")


def _bind(path):
    lib = ctypes.CDLL(path)
    lib.gdla_oracle_prefill_rows.restype = ctypes.c_int
    lib.gdla_oracle_prefill_rows.argtypes = [
        _f32p, _f32p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ctypes.c_int, ctypes.c_int, ctypes.c_double, ctypes.c_long, _i32p, _i32p,
        _f32p, _f32p, _f32p, _f32p, _f64p]
    lib.gdla_oracle_decode.restype = ctypes.c_int
    lib.gdla_oracle_decode.argtypes = [
        _f32p, _f32p, _f32p, _f32p, _i32p, _f32p, _f32p, ctypes.c_int, ctypes.c_int,
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_double, _f64p]
    lib.gdla_oracle_decode_latent.restype = ctypes.c_int
    lib.gdla_oracle_decode_latent.argtypes = [
        _f32p, _f32p, _f32p, _f32p, _f32p, _i32p, _f32p, _f32p, ctypes.c_int, ctypes.c_int,
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ctypes.c_double, _f64p]
    lib.gdla_oracle_prep.restype = ctypes.c_int
    lib.gdla_oracle_prep.argtypes = [
        _f32p, _f32p, _f32p, _f32p, _f32p, _f32p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_double,
        _f64p, _f64p, _f64p, _f64p, _f64p]
    lib.gdla_oracle_num_threads.restype = ctypes.c_int
    lib.gdla_oracle_num_threads.argtypes = []
    lib.gdla_oracle_set_threads.restype = None
    lib.gdla_oracle_set_threads.argtypes = [ctypes.c_int]
    return lib


def library(path=None):
    """The loaded oracle library (built with gcc on first use if missing)."""
    global _LIB
    if path is not None:
        return _bind(path)
    if _LIB is None:
        if not os.path.exists(_build.LIBRARY):
            _build.build_oracle()
        _LIB = _bind(_build.LIBRARY)
    return _LIB


_LIB_FP32 = None


def library_fp32():
    """The fp32 build of the same source (built with gcc on first use if
    missing): every prefill and decode product, sum and exponential in fp32."""
    global _LIB_FP32
    if _LIB_FP32 is None:
        if not os.path.exists(_build.LIBRARY_FP32):
            _build.build_oracle(fp32=True)
        _LIB_FP32 = _bind(_build.LIBRARY_FP32)
    return _LIB_FP32


def num_threads(lib=None):
    """OpenMP threads the oracle's parallel loops use on this host."""
    return int((lib or library()).gdla_oracle_num_threads())


def set_threads(n, lib=None):
    """Threads for the oracle's later parallel loops (the build's own OpenMP
    runtime; n >= 1)."""
    (lib or library()).gdla_oracle_set_threads(int(n))


def _f32(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float32))


def prefill_rows(k, v, q_signal_rows, q_noise_rows, lam_rows, gate_rows, row_b, row_t,
                 window=0, scale=None, T=None, lib=None):
    """Output rows O[b_r, t_r] for the listed query positions.

    k [B,T,n_kv,d_qk], v [B,T,n_kv,d_v]; per-row inputs
    q_signal_rows [R,n_kv*g,d_qk], q_noise_rows [R,n_kv,d_qk],
    lam_rows [R,n_kv*g], gate_rows [R,n_kv*g,d_v]; returns float64 [R,n_kv*g,d_v].
    """
    k = _f32(k)
    v = _f32(v)
    B, Tk, n_kv, d_qk = k.shape
    d_v = v.shape[3]
    qs = _f32(q_signal_rows)
    R = qs.shape[0]
    group = qs.shape[1] // n_kv
    if scale is None:
        scale = 1.0 / np.sqrt(d_qk)
    out = np.empty((R, n_kv * group, d_v), dtype=np.float64)
    rb = np.ascontiguousarray(np.asarray(row_b, dtype=np.int32))
    rt = np.ascontiguousarray(np.asarray(row_t, dtype=np.int32))
    L = lib if lib is not None else library()
    rc = L.gdla_oracle_prefill_rows(k, v, B, Tk, n_kv, group, d_qk, d_v, int(window),
                                    float(scale), R, rb, rt, qs, _f32(q_noise_rows),
                                    _f32(lam_rows), _f32(gate_rows), out)
    if rc != 0:
        raise ValueError("oracle prefill rejected its arguments (code %d)" % rc)
    return out


def prefill(q_signal, q_noise, k, v, lam, gate, window=0, scale=None, lib=None):
    """Full prefill: q_signal [B,T,n_kv*g,d_qk] ... -> float64 [B,T,n_kv*g,d_v]."""
    qs = _f32(q_signal)
    B, T, n_sig, d_qk = qs.shape
    d_v = np.asarray(v).shape[3]
    bb, tt = np.meshgrid(np.arange(B, dtype=np.int32), np.arange(T, dtype=np.int32),
                         indexing="ij")
    out = prefill_rows(k, v, qs.reshape(B * T, n_sig, d_qk),
                       _f32(q_noise).reshape(B * T, -1, d_qk),
                       _f32(lam).reshape(B * T, n_sig),
                       _f32(gate).reshape(B * T, n_sig, d_v),
                       bb.reshape(-1), tt.reshape(-1), window=window, scale=scale, lib=lib)
    return out.reshape(B, T, n_sig, d_v)


def decode(q_signal, q_noise, k_cache, v_cache, cu_seqlens, lam, gate, window=0,
           scale=None, lib=None):
    """Decode: q_signal [B,n_kv*g,d_qk], caches [total,n_kv,d] -> float64 [B,n_kv*g,d_v]."""
    qs = _f32(q_signal)
    B, n_sig, d_qk = qs.shape
    kc = _f32(k_cache)
    vc = _f32(v_cache)
    n_kv = kc.shape[1]
    d_v = vc.shape[2]
    group = n_sig // n_kv
    if scale is None:
        scale = 1.0 / np.sqrt(d_qk)
    out = np.empty((B, n_sig, d_v), dtype=np.float64)
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
    L = lib if lib is not None else library()
    rc = L.gdla_oracle_decode(qs, _f32(q_noise), kc, vc, cu, _f32(lam), _f32(gate), B, n_kv,
                              group, d_qk, d_v, int(window), float(scale), out)
    if rc != 0:
        raise ValueError("oracle decode rejected its arguments (code %d)" % rc)
    return out


def decode_latent(q_signal, q_noise, latent, w_uk, w_uv, cu_seqlens, lam, gate, window=0,
                  scale=None, lib=None):
    """Decode over a latent cache.

    latent [total, d_c + d_r] (compressed KV, then the shared rotary key),
    w_uk [n_kv, d_kc, d_c], w_uv [n_kv, d_v, d_c], q_signal [B, n_kv*g, d_kc + d_r],
    q_noise [B, n_kv, d_kc + d_r] -> float64 [B, n_kv*g, d_v].
    """
    qs = _f32(q_signal)
    B, n_sig, d_qk = qs.shape
    wk = _f32(w_uk)
    wv = _f32(w_uv)
    n_kv, d_kc, d_c = wk.shape
    d_v = wv.shape[1]
    d_r = d_qk - d_kc
    lat = _f32(latent)
    assert lat.shape[1] == d_c + d_r, lat.shape
    group = n_sig // n_kv
    if scale is None:
        scale = 1.0 / np.sqrt(d_qk)
    out = np.empty((B, n_sig, d_v), dtype=np.float64)
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
    L = lib if lib is not None else library()
    rc = L.gdla_oracle_decode_latent(qs, _f32(q_noise), lat, wk, wv, cu, _f32(lam), _f32(gate), B,
                                     n_kv, group, d_c, d_r, d_kc, d_v, int(window), float(scale),
                                     out)
    if rc != 0:
        raise ValueError("oracle latent decode rejected its arguments (code %d)" % rc)
    return out


def prep(q_signal, q_noise, k_rope, x, w_lambda, gate_pre, pos0=0, theta=10000.0, lib=None):
    """The step ahead of the attention core.

    q_signal [B, T, n_sig, d_qk], q_noise [B, T, n_kv, d_qk], k_rope [B, T, 64],
    x [B, T, d_model], w_lambda [n_sig, d_model], gate_pre [B, T, n_sig, d_v]
    -> dict of float64 arrays: q_signal, q_noise (rotary parts rotated), k_rot
    [B, T, n_kv, 64] (the rotated shared key as it lands in each KV head), lam
    [B, T, n_sig] and gate [B, T, n_sig, d_v].
    """
    qs, qn, kr = _f32(q_signal), _f32(q_noise), _f32(k_rope)
    xx, wl, gp = _f32(x), _f32(w_lambda), _f32(gate_pre)
    B, T, n_sig, d_qk = qs.shape
    n_kv = qn.shape[2]
    d_model = xx.shape[2]
    d_v = gp.shape[3]
    assert kr.shape == (B, T, 64) and wl.shape == (n_sig, d_model), (kr.shape, wl.shape)
    out = {"q_signal": np.empty(qs.shape, np.float64), "q_noise": np.empty(qn.shape, np.float64),
           "k_rot": np.empty((B, T, n_kv, 64), np.float64), "lam": np.empty((B, T, n_sig), np.float64),
           "gate": np.empty(gp.shape, np.float64)}
    L = lib if lib is not None else library()
    rc = L.gdla_oracle_prep(qs, qn, kr, xx, wl, gp, B, T, n_kv, n_sig // n_kv, d_qk, d_v, d_model,
                            int(pos0), float(theta), out["q_signal"], out["q_noise"], out["k_rot"],
                            out["lam"], out["gate"])
    if rc != 0:
        raise ValueError("oracle prep rejected its arguments (code %d)" % rc)
    return out
