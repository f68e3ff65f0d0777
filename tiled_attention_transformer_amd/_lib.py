"""ctypes loading of ``libattn.so`` with the signatures of include/attn.h."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libattn.so")

_p, _i, _f, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t

# name -> (restype, argtypes); mirrors include/attn.h
SIGNATURES = {
    "attn_fwd": (_i, [_p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _f, _i, _p]),
    "attn_fwd_exp2_poly": (_i, [_p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _f, _i, _i, _p]),
    "attn_fwd_varlen": (_i, [_p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _i, _f,
                             _i, _p]),
    "attn_fwd_splitkv": (_i, [_p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _f, _i, _i, _p, _sz, _p]),
    "attn_fwd_splitkv_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i, _i]),
    "attn_varlen_check": (_i, [_p, _i, _i, _p]),
    "attn_decode": (_i, [_p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _f, _i, _p, _sz, _p]),
    "attn_decode_noalloc": (_i, [_p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _f, _i, _p]),
    "attn_decode_varlen": (_i, [_p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _f, _i, _p, _sz,
                                _p]),
    "attn_decode_paged": (_i, [_p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _f, _i,
                               _p, _sz, _p]),
    "attn_decode_fp8": (_i, [_p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _f, _f, _f, _i, _p, _sz,
                             _p]),
    "attn_kmeans_assign": (_i, [_p, _p, _p, _p, _i, _i, _i, _p]),
    "attn_decode_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i]),
    "attn_decode_varlen_workspace_bytes": (_sz, [_i, _i, _i, _i, _i]),
    "attn_decode_pick_splits": (_i, [_i, _i, _i, _i]),
    "attn_status_string": (ctypes.c_char_p, [_i]),
}

_lib = None


def load():
    """Load the built library; raise if it has not been built (no fallback)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                "libattn.so is not built (expected at %s); build it with "
                "`python -m tiled_attention_transformer_amd.build` or "
                "__graft_entry__.build()" % LIB_PATH)
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib
