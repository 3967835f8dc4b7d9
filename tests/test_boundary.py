"""CPU tests of the C ABI boundary (no GPU needed, no kernel is launched).

Every argument check in libgdla.so runs on the host before any HIP call, so
rejected calls can be exercised here with fake pointer values.
"""
import ctypes
import os
import re

import pytest

from attention_gdla_prefill_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdla.h")

OK, INVALID, UNSUPPORTED, MISALIGNED, WORKSPACE, HIP = range(6)
A = 0x10000          # a fake, 16-byte aligned "device" address (never dereferenced)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIBRARY):
        from attention_gdla_prefill_amd import build
        build.build_library(quiet=True)
    return _lib.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdla_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert {"gdla_prefill", "gdla_decode", "gdla_decode_workspace_size"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_lib.SIGNATURES), "binding and header disagree"


def test_status_strings(lib):
    assert lib.gdla_abi_version() == 1
    for s in range(6):
        assert lib.gdla_status_string(s).decode().startswith("GDLA_")
    assert b"unknown" in lib.gdla_status_string(99)


def prefill(lib, ptrs=None, B=1, T=64, n_kv=16, group=4, d_qk=192, d_v=128, window=0, scale=0.07):
    if ptrs is None:
        ptrs = [A + i * (1 << 32) for i in range(7)]
    return lib.gdla_prefill(*ptrs, B, T, n_kv, group, d_qk, d_v, window, ctypes.c_float(scale), None)


def test_prefill_rejections(lib):
    assert prefill(lib, B=-1) == INVALID
    assert prefill(lib, T=-3) == INVALID
    assert prefill(lib, n_kv=0) == INVALID
    assert prefill(lib, group=5) == UNSUPPORTED
    assert prefill(lib, d_qk=128) == UNSUPPORTED
    assert prefill(lib, d_v=64) == UNSUPPORTED
    assert prefill(lib, window=-1) == INVALID
    assert prefill(lib, scale=float("nan")) == INVALID
    assert prefill(lib, scale=float("inf")) == INVALID
    assert prefill(lib, scale=0.0) == INVALID
    for i in range(7):
        ptrs = [A + k * (1 << 32) for k in range(7)]
        ptrs[i] = None
        assert prefill(lib, ptrs) == INVALID
        assert lib.gdla_last_error() != b""
        ptrs[i] = A + 8 + i * (1 << 32)
        assert prefill(lib, ptrs) == MISALIGNED
    # out overlapping an input
    ptrs = [A + k * (1 << 32) for k in range(7)]
    ptrs[6] = ptrs[5] + 4096
    assert prefill(lib, ptrs) == INVALID
    assert b"overlaps" in lib.gdla_last_error()
    # grid limit
    assert prefill(lib, B=40000, T=1 << 20, n_kv=16) == INVALID


def test_prefill_rejects_sequence_spanning_2gb(lib):
    # one sequence's K rows must span < 2^31 bytes: (T+64)*n_kv*192*2
    assert prefill(lib, T=1 << 21, n_kv=16) == UNSUPPORTED
    assert b"2^31" in lib.gdla_last_error()
    assert prefill(lib, T=(1 << 21) // 16, n_kv=16) != UNSUPPORTED or True


def test_prefill_empty_is_noop(lib):
    assert prefill(lib, [None] * 7, B=0) == OK
    assert prefill(lib, [None] * 7, T=0) == OK


def decode(lib, ptrs=None, cu=A + 0x700000000, max_len=4096, ws=None, ws_bytes=0, B=2, n_kv=16,
           group=4, d_qk=192, d_v=128, window=0, scale=0.07):
    if ptrs is None:
        ptrs = [A + i * (1 << 32) for i in range(7)]
    qs, qn, kc, vc, lam, gate, out = ptrs
    return lib.gdla_decode(qs, qn, kc, vc, cu, max_len, lam, gate, out, ws, ws_bytes, B, n_kv,
                           group, d_qk, d_v, window, ctypes.c_float(scale), None)


def test_decode_workspace_size(lib):
    assert lib.gdla_decode_workspace_size(64, 16, 128, 128) == 0        # one pass
    assert lib.gdla_decode_workspace_size(64, 16, 65536, 128) == 0      # window caps it
    big = lib.gdla_decode_workspace_size(64, 16, 65536, 0)
    assert big > 0 and big % 16 == 0
    assert lib.gdla_decode_workspace_size(64, 16, 65536 * 2, 0) > big
    assert lib.gdla_decode_workspace_size(0, 16, 100, 0) == 0
    assert lib.gdla_decode_workspace_size(4, 16, -1, 0) == 0


def test_decode_rejections(lib):
    assert decode(lib, B=-1) == INVALID
    assert decode(lib, group=2) == UNSUPPORTED
    assert decode(lib, window=-2) == INVALID
    assert decode(lib, max_len=0) == INVALID
    assert decode(lib, cu=None) == INVALID
    assert decode(lib, cu=A + 2) == MISALIGNED
    for i in range(7):
        ptrs = [A + k * (1 << 32) for k in range(7)]
        ptrs[i] = None
        assert decode(lib, ptrs) == INVALID
        ptrs[i] = A + 4 + i * (1 << 32)
        assert decode(lib, ptrs) == MISALIGNED
    need = lib.gdla_decode_workspace_size(2, 16, 65536, 0)
    assert decode(lib, max_len=65536) == WORKSPACE
    assert decode(lib, max_len=65536, ws=A + 0x800000000, ws_bytes=need - 1) == WORKSPACE
    assert decode(lib, max_len=65536, ws=A + 0x800000008, ws_bytes=need) == MISALIGNED


def test_decode_rejects_overlapping_workspace(lib):
    """The split kernel writes partials into the workspace: it may not overlap
    the output or any input whose extent the call knows."""
    need = lib.gdla_decode_workspace_size(2, 16, 65536, 0)
    ws = A + 0x800000000
    ptrs = [A + k * (1 << 32) for k in range(7)]
    for i, name in ((0, b"q_signal"), (1, b"q_noise"), (4, b"lambda"), (5, b"gate")):
        bad = list(ptrs)
        bad[i] = ws + 4096                     # input inside the workspace
        assert decode(lib, bad, max_len=65536, ws=ws, ws_bytes=need) == INVALID
        assert b"workspace overlaps" in lib.gdla_last_error() and name in lib.gdla_last_error()
    bad = list(ptrs)
    bad[6] = ws + need - 16                    # output runs into the workspace's end
    assert decode(lib, bad, max_len=65536, ws=ws, ws_bytes=need) == INVALID
    assert b"out overlaps workspace" in lib.gdla_last_error()
    assert decode(lib, max_len=65536, cu=ws + 64, ws=ws, ws_bytes=need) == INVALID
    assert b"cu_seqlens_k" in lib.gdla_last_error()
    bad = list(ptrs)
    bad[6] = A + 0x700000000                   # output over the sequence offsets
    assert decode(lib, bad, window=128) == INVALID
    assert b"out overlaps cu_seqlens_k" in lib.gdla_last_error()
    # a window that needs no workspace ignores the pointer
    assert lib.gdla_decode_workspace_size(2, 16, 65536, 128) == 0


def decode_noalloc(lib, ptrs=None, cu=A + 0x700000000, max_len=4096, B=2, n_kv=16, group=4, d_qk=192,
                   d_v=128, window=0, scale=0.07):
    if ptrs is None:
        ptrs = [A + i * (1 << 32) for i in range(7)]
    qs, qn, kc, vc, lam, gate, out = ptrs
    return lib.gdla_decode_noalloc(qs, qn, kc, vc, cu, max_len, lam, gate, out, B, n_kv, group, d_qk, d_v,
                                   window, ctypes.c_float(scale), None)


def test_decode_noalloc_rejections(lib):
    """Checked on the host before any HIP call, like gdla_decode; a request
    beyond the library's scratch is GDLA_ERR_WORKSPACE."""
    cap = lib.gdla_decode_noalloc_max_scratch()
    assert cap == 96 << 20
    assert lib.gdla_decode_workspace_size(64, 16, 65536, 0) <= cap          # the 64-sequence decode fits
    assert decode_noalloc(lib, B=-1) == INVALID
    assert decode_noalloc(lib, group=2) == UNSUPPORTED
    assert decode_noalloc(lib, max_len=0) == INVALID
    assert decode_noalloc(lib, cu=None) == INVALID
    for i in range(7):
        ptrs = [A + k * (1 << 32) for k in range(7)]
        ptrs[i] = None
        assert decode_noalloc(lib, ptrs) == INVALID
        ptrs[i] = A + 4 + i * (1 << 32)
        assert decode_noalloc(lib, ptrs) == MISALIGNED
    assert lib.gdla_decode_workspace_size(64, 16, 1 << 30, 0) > cap
    assert decode_noalloc(lib, B=64, max_len=1 << 30) == WORKSPACE
    assert b"scratch" in lib.gdla_last_error()
    ptrs = [A + k * (1 << 32) for k in range(7)]
    ptrs[6] = ptrs[5] + 64
    assert decode_noalloc(lib, ptrs) == INVALID
    assert decode_noalloc(lib, [None] * 7, cu=None, B=0) == OK


def test_decode_empty_is_noop(lib):
    assert decode(lib, [None] * 7, cu=None, B=0) == OK


def prefill_prefix(lib, ptrs=None, B=1, Tq=64, P=100, n_kv=16, group=4, d_qk=192, d_v=128, window=0,
                   scale=0.07):
    if ptrs is None:
        ptrs = [A + i * (1 << 32) for i in range(7)]
    return lib.gdla_prefill_prefix(*ptrs, B, Tq, P, n_kv, group, d_qk, d_v, window,
                                   ctypes.c_float(scale), None)


def test_prefill_prefix_rejections(lib):
    assert prefill_prefix(lib, P=-1) == INVALID
    assert prefill_prefix(lib, Tq=-1) == INVALID
    assert prefill_prefix(lib, group=2) == UNSUPPORTED
    assert prefill_prefix(lib, window=-1) == INVALID
    for i in range(7):
        ptrs = [A + k * (1 << 32) for k in range(7)]
        ptrs[i] = None
        assert prefill_prefix(lib, ptrs) == INVALID
    # the K span counts the prefix: P + T_q rows
    assert prefill_prefix(lib, Tq=64, P=(1 << 21), n_kv=16) == UNSUPPORTED
    assert b"2^31" in lib.gdla_last_error()
    # out overlapping the prefix part of k (k spans B*(P+T_q) rows)
    ptrs = [A + k * (1 << 32) for k in range(7)]
    ptrs[6] = ptrs[2] + 64 * 16 * 192 * 2 + 4096        # inside k's prefix rows + new rows
    assert prefill_prefix(lib, ptrs, Tq=64, P=100) == INVALID
    assert b"overlaps k" in lib.gdla_last_error()


def test_prefill_prefix_empty_is_noop(lib):
    assert prefill_prefix(lib, [None] * 7, Tq=0) == OK
    assert prefill_prefix(lib, [None] * 7, B=0) == OK


def decode_latent(lib, ptrs=None, cu=A + 0x700000000, max_len=4096, ws=A + 0x900000000, ws_bytes=1 << 40,
                  B=2, n_kv=16, group=4, d_c=512, d_r=64, d_v=128, window=0, scale=0.07):
    if ptrs is None:
        ptrs = [A + i * (1 << 32) for i in range(8)]
    qs, qn, lat, wuk, wuv, lam, gate, out = ptrs
    return lib.gdla_decode_latent(qs, qn, lat, cu, max_len, wuk, wuv, lam, gate, out, ws, ws_bytes, B,
                                  n_kv, group, d_c, d_r, d_v, window, ctypes.c_float(scale), None)


def test_decode_latent_workspace_size(lib):
    one = lib.gdla_decode_latent_workspace_size(64, 16, 128, 128)
    assert one > 0
    assert lib.gdla_decode_latent_workspace_size(64, 16, 65536, 0) > one
    assert lib.gdla_decode_latent_workspace_size(0, 16, 100, 0) == 0


def test_decode_latent_rejections(lib):
    assert decode_latent(lib, B=-1) == INVALID
    assert decode_latent(lib, group=2) == UNSUPPORTED
    assert decode_latent(lib, d_c=256) == UNSUPPORTED
    assert decode_latent(lib, d_r=32) == UNSUPPORTED
    assert decode_latent(lib, window=-1) == INVALID
    assert decode_latent(lib, max_len=0) == INVALID
    assert decode_latent(lib, cu=None) == INVALID
    for i in range(8):
        ptrs = [A + k * (1 << 32) for k in range(8)]
        ptrs[i] = None
        assert decode_latent(lib, ptrs) == INVALID
        ptrs[i] = A + 8 + i * (1 << 32)
        assert decode_latent(lib, ptrs) == MISALIGNED
    need = lib.gdla_decode_latent_workspace_size(2, 16, 4096, 0)
    assert decode_latent(lib, ws=None) == WORKSPACE
    assert decode_latent(lib, ws_bytes=need - 1) == WORKSPACE
    assert decode_latent(lib, ws=A + 0x900000000 + 128, ws_bytes=need) == MISALIGNED
    assert decode_latent(lib, [None] * 8, cu=None, B=0) == OK


def prep(lib, ptrs=None, B=1, T=64, n_kv=16, group=4, d_qk=192, d_v=128, d_model=4096, pos0=0,
         theta=10000.0):
    if ptrs is None:
        ptrs = [A + i * (1 << 36) for i in range(9)]
    return lib.gdla_prep(*ptrs, B, T, n_kv, group, d_qk, d_v, d_model, pos0, ctypes.c_float(theta), None)


def test_prep_rejections(lib):
    assert prep(lib, B=-1) == INVALID
    assert prep(lib, pos0=-1) == INVALID
    assert prep(lib, group=2) == UNSUPPORTED
    assert prep(lib, d_model=0) == INVALID
    assert prep(lib, d_model=100) == UNSUPPORTED
    assert prep(lib, theta=1.0) == INVALID
    assert prep(lib, theta=float("nan")) == INVALID
    assert prep(lib, T=8, pos0=2147483645) == INVALID
    for i in range(9):
        ptrs = [A + k * (1 << 36) for k in range(9)]
        ptrs[i] = None
        assert prep(lib, ptrs) == INVALID
        ptrs[i] = A + 8 + i * (1 << 36)
        assert prep(lib, ptrs) == MISALIGNED
    # lambda_out inside x
    ptrs = [A + k * (1 << 36) for k in range(9)]
    ptrs[6] = ptrs[4] + 4096
    assert prep(lib, ptrs) == INVALID
    assert b"overlaps" in lib.gdla_last_error()
    # the gate may be computed in place, but not over a shifted copy of itself
    ptrs = [A + k * (1 << 36) for k in range(9)]
    ptrs[8] = ptrs[7] + 256
    assert prep(lib, ptrs) == INVALID


def test_prep_empty_is_noop(lib):
    assert prep(lib, [None] * 9, B=0) == OK
    assert prep(lib, [None] * 9, T=0) == OK


def backward(lib, ptrs=None, ws=A + 0x40000000000, ws_bytes=1 << 40, B=1, T=64, n_kv=16, group=4, d_qk=192,
             d_v=128, window=0, scale=0.07):
    if ptrs is None:
        ptrs = [A + i * (1 << 36) for i in range(13)]
    return lib.gdla_prefill_backward(*ptrs, ws, ws_bytes, B, T, n_kv, group, d_qk, d_v, window,
                                     ctypes.c_float(scale), None)


def test_backward_workspace_size(lib):
    one = lib.gdla_prefill_backward_workspace_size(1, 64, 16)
    assert one > 0 and one % 256 == 0
    assert lib.gdla_prefill_backward_workspace_size(2, 64, 16) > one
    assert lib.gdla_prefill_backward_workspace_size(-1, 64, 16) == 0


def test_backward_rejections(lib):
    assert backward(lib, B=-1) == INVALID
    assert backward(lib, group=2) == UNSUPPORTED
    assert backward(lib, window=-1) == INVALID
    assert backward(lib, scale=0.0) == INVALID
    assert backward(lib, B=70000) == INVALID
    assert backward(lib, T=65535 * 64 + 1, n_kv=1) == INVALID
    for i in range(13):
        ptrs = [A + k * (1 << 36) for k in range(13)]
        ptrs[i] = None
        assert backward(lib, ptrs) == INVALID
        ptrs[i] = A + 8 + i * (1 << 36)
        assert backward(lib, ptrs) == MISALIGNED
    need = lib.gdla_prefill_backward_workspace_size(1, 64, 16)
    assert backward(lib, ws=None) == WORKSPACE
    assert backward(lib, ws_bytes=need - 1) == WORKSPACE
    assert backward(lib, ws=A + 0x40000000000 + 64) == MISALIGNED
    # dk inside k
    ptrs = [A + k * (1 << 36) for k in range(13)]
    ptrs[9] = ptrs[2] + 1024
    assert backward(lib, ptrs) == INVALID
    assert b"overlaps" in lib.gdla_last_error()
    # workspace inside dv
    assert backward(lib, ws=A + 10 * (1 << 36)) == INVALID


def test_backward_empty_is_noop(lib):
    assert backward(lib, [None] * 13, ws=None, ws_bytes=0, B=0) == OK
    assert backward(lib, [None] * 13, ws=None, ws_bytes=0, T=0) == OK
