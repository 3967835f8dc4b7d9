"""CPU tests of the Python binding's host logic (no kernel runs): with
GDLA_SYNC_CHECK=1 every entry point waits for the device after its launch,
and without it none does.  The C library is replaced by a stand-in that
accepts every call, and tensor metadata checks are bypassed, so only the
binding's own control flow is exercised."""
import pytest
import torch

import attention_gdla_prefill_amd as gdla
from attention_gdla_prefill_amd import _lib, api


class _FakeLib:
    def __getattr__(self, name):
        return lambda *args: 0


def _calls():
    z = lambda *shape: torch.zeros(shape, dtype=torch.bfloat16)
    i32 = torch.zeros(3, dtype=torch.int32)
    B, T, kv = 1, 2, 1
    s = 4 * kv
    return {
        "prefill": lambda: api.prefill(z(B, T, s, 192), z(B, T, kv, 192), z(B, T, kv, 192), z(B, T, kv, 128),
                                       z(B, T, s), z(B, T, s, 128), out=z(B, T, s, 128)),
        "prefill_prefix": lambda: api.prefill_prefix(z(B, 1, s, 192), z(B, 1, kv, 192), z(B, T, kv, 192),
                                                     z(B, T, kv, 128), z(B, 1, s), z(B, 1, s, 128),
                                                     out=z(B, 1, s, 128)),
        "decode": lambda: api.decode(z(2, s, 192), z(2, kv, 192), z(5, kv, 192), z(5, kv, 128), i32, 3, z(2, s),
                                     z(2, s, 128), out=z(2, s, 128), workspace=torch.zeros(16, dtype=torch.uint8)),
        "decode_noalloc": lambda: api.decode_noalloc(z(2, s, 192), z(2, kv, 192), z(5, kv, 192), z(5, kv, 128),
                                                     i32, 3, z(2, s), z(2, s, 128), out=z(2, s, 128)),
        "decode_latent": lambda: api.decode_latent(z(2, s, 192), z(2, kv, 192), z(5, 576), i32, 3,
                                                   z(kv, 128, 512), z(kv, 128, 512), z(2, s), z(2, s, 128),
                                                   out=z(2, s, 128), workspace=torch.zeros(256, dtype=torch.uint8)),
        "prep": lambda: api.prep(z(B, T, s, 192), z(B, T, kv, 192), z(B, T, 64), z(B, T, kv, 192), z(B, T, 32),
                                 z(s, 32), z(B, T, s, 128), lam_out=z(B, T, s), gate_out=z(B, T, s, 128)),
        "prefill_backward": lambda: api.prefill_backward(z(B, T, s, 192), z(B, T, kv, 192), z(B, T, kv, 192),
                                                         z(B, T, kv, 128), z(B, T, s), z(B, T, s, 128),
                                                         z(B, T, s, 128), workspace=torch.zeros(256, dtype=torch.uint8)),
    }


@pytest.fixture
def stubbed(monkeypatch):
    syncs = []
    monkeypatch.setattr(_lib, "load", lambda path=None: _FakeLib())
    monkeypatch.setattr(api, "_check", lambda *a, **k: None)
    monkeypatch.setattr(api, "_stream_ptr", lambda device: None)
    monkeypatch.setattr(torch.cuda, "synchronize", lambda device=None: syncs.append(device))
    return syncs


@pytest.mark.parametrize("name", sorted(_calls()))
def test_sync_check_waits_after_every_launch(stubbed, monkeypatch, name):
    monkeypatch.setenv("GDLA_SYNC_CHECK", "1")
    _calls()[name]()
    assert len(stubbed) == 1, stubbed


@pytest.mark.parametrize("value", ["", "0"])
def test_no_wait_without_sync_check(stubbed, monkeypatch, value):
    monkeypatch.setenv("GDLA_SYNC_CHECK", value)
    for call in _calls().values():
        call()
    assert stubbed == []


def test_every_entry_point_is_covered():
    public = {n for n in gdla.__all__} if hasattr(gdla, "__all__") else {
        n for n in dir(api) if not n.startswith("_") and callable(getattr(api, n))}
    launchers = {n for n in public if n in ("prefill", "prefill_prefix", "decode", "decode_noalloc", "decode_latent",
                                            "prep", "prefill_backward")}
    assert launchers == set(_calls())
