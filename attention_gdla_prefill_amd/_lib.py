"""ctypes loader for libgdla.so, the C ABI declared in include/gdla.h.

There is no fallback: if the HIP library has not been built, loading raises.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(HERE, "libgdla.so")

# Every symbol include/gdla.h declares, with its ctypes signature.
_P = ctypes.c_void_p
_I = ctypes.c_int
SIGNATURES = {
    "gdla_abi_version": (_I, []),
    "gdla_status_string": (ctypes.c_char_p, [_I]),
    "gdla_last_error": (ctypes.c_char_p, []),
    "gdla_prefill": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I,
                          ctypes.c_float, _P]),
    "gdla_prefill_prefix": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I,
                                 ctypes.c_float, _P]),
    "gdla_decode_workspace_size": (ctypes.c_size_t, [_I, _I, _I, _I]),
    "gdla_decode": (_I, [_P, _P, _P, _P, _P, _I, _P, _P, _P, _P, ctypes.c_size_t,
                         _I, _I, _I, _I, _I, _I, ctypes.c_float, _P]),
    "gdla_decode_noalloc_max_scratch": (ctypes.c_size_t, []),
    "gdla_decode_noalloc": (_I, [_P, _P, _P, _P, _P, _I, _P, _P, _P, _I, _I, _I, _I, _I, _I,
                                 ctypes.c_float, _P]),
    "gdla_decode_latent_workspace_size": (ctypes.c_size_t, [_I, _I, _I, _I]),
    "gdla_decode_latent": (_I, [_P, _P, _P, _P, _I, _P, _P, _P, _P, _P, _P, ctypes.c_size_t,
                                _I, _I, _I, _I, _I, _I, _I, ctypes.c_float, _P]),
    "gdla_prefill_backward_workspace_size": (ctypes.c_size_t, [_I, _I, _I]),
    "gdla_prefill_backward": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t,
                                   _I, _I, _I, _I, _I, _I, _I, ctypes.c_float, _P]),
    "gdla_prep": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I,
                       ctypes.c_float, _P]),
}

_lib = None


def load(path=None):
    """Load (once) and return the library; raises OSError if it is not built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIBRARY
    if not os.path.exists(p):
        raise OSError("libgdla.so is not built (%s); run __graft_entry__.build() or "
                      "python attention_gdla_prefill_amd/build.py" % p)
    lib = ctypes.CDLL(p)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _lib = lib
    return lib


class GdlaError(RuntimeError):
    def __init__(self, status, detail):
        self.status = status
        super().__init__("%s (%s)" % (detail, status_string(status)))


def status_string(status):
    return load().gdla_status_string(int(status)).decode()


def check(status):
    if status != 0:
        raise GdlaError(status, load().gdla_last_error().decode())


def sync_check_enabled():
    """GDLA_SYNC_CHECK set to anything but "" or "0"."""
    return os.environ.get("GDLA_SYNC_CHECK", "") not in ("", "0")


def after_launch(device):
    """Called after every launch: with GDLA_SYNC_CHECK=1 it waits for the
    device, which raises any asynchronous HIP error there and then."""
    if sync_check_enabled():
        import torch
        torch.cuda.synchronize(device)
