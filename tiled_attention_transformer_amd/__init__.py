"""Fused tiled attention forward for AMD MI355X (gfx950).

The computation lives in hand-written HIP kernels behind a C ABI
(``libattn.so``, declared in include/attn.h); this package is the thin
binding.  Import the functions from :mod:`tiled_attention_transformer_amd.api`
(they need torch with a ROCm GPU for device memory and streams).
"""
from ._lib import LIB_PATH, load  # noqa: F401

__all__ = ["LIB_PATH", "load"]
