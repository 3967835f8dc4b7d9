"""GDLA attention core (Grouped Differential Latent Attention) for MI355X / gfx950.

The computation lives in hand-written HIP kernels behind the C ABI of
include/gdla.h (libgdla.so); this package is its Python binding.
"""
from .api import (decode, decode_latent, decode_latent_workspace_size, decode_noalloc,  # noqa: F401
                  decode_noalloc_max_scratch, decode_workspace_size, prefill, prefill_backward,
                  prefill_backward_workspace_size, prefill_prefix, prep)
from ._lib import GdlaError  # noqa: F401
