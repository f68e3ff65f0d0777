"""Thin Python binding of the attention C ABI (include/attn.h).

Each function has the name of the C entry point it calls and only marshals
arguments: it reads sizes off the torch tensors, allocates missing outputs
with torch (device memory is plumbing here), passes raw device pointers and
the current stream, and raises :class:`AttnError` on a nonzero status.  Every
step of the computation runs in the HIP kernels of ``libattn.so``; there is
no other code path.
"""
from __future__ import annotations

import ctypes
import math

import torch

from . import _lib

ATTN_OK = 0
STATUS_NAMES = {
    0: "ATTN_OK", 1: "ATTN_ERR_NULLPTR", 2: "ATTN_ERR_SHAPE", 3: "ATTN_ERR_UNSUPPORTED_D",
    4: "ATTN_ERR_GQA_RATIO", 5: "ATTN_ERR_ALIGNMENT", 6: "ATTN_ERR_WORKSPACE",
    7: "ATTN_ERR_SEQLENS", 8: "ATTN_ERR_HIP", 9: "ATTN_ERR_SCALE", 10: "ATTN_ERR_SCRATCH_LIMIT",
}


class AttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        text = _lib.load().attn_status_string(status).decode()
        super().__init__("%s: %s (%s)" % (where, STATUS_NAMES.get(status, status), text))


def _check(status: int, where: str):
    if status != ATTN_OK:
        raise AttnError(status, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _need(t, name, dtype, ndim):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if t.device.type != "cuda":
        raise ValueError("%s must be on the GPU" % name)
    if t.dim() != ndim:
        raise ValueError("%s must have %d dimensions, got %s" % (name, ndim, tuple(t.shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _scale(scale, d):
    return float(1.0 / math.sqrt(d)) if scale is None else float(scale)


def attn_status_string(status: int) -> str:
    return _lib.load().attn_status_string(int(status)).decode()


def attn_fwd(q, k, v, o=None, lse=None, scale=None, causal=False, want_lse=True, stream=None):
    """Attention forward over a fixed batch; returns ``(o, lse)``.

    q ``[B,Sq,Hq,d]``, k/v ``[B,Skv,Hkv,d]`` bf16 on the GPU; o like q (bf16),
    lse ``[B,Hq,Sq]`` fp32 (``None`` when ``want_lse`` is false and no lse is
    given).  scale defaults to 1/sqrt(d).
    """
    return _fwd(q, k, v, o, lse, scale, causal, want_lse, stream, None)


def attn_fwd_exp2_poly(q, k, v, poly_per_32, o=None, lse=None, scale=None, causal=False,
                       want_lse=True, stream=None):
    """``attn_fwd`` with ``poly_per_32`` (0, 4, 8 or 16) of each lane's 32
    exponentials per key tile computed by the library's exp2 polynomial."""
    return _fwd(q, k, v, o, lse, scale, causal, want_lse, stream, int(poly_per_32))


def _fwd(q, k, v, o, lse, scale, causal, want_lse, stream, poly):
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, torch.bfloat16, 4)
    B, Sq, Hq, d = q.shape
    Skv, Hkv = k.shape[1], k.shape[2]
    if tuple(v.shape) != tuple(k.shape) or k.shape[0] != B or k.shape[3] != d:
        raise ValueError("shape mismatch: q %s k %s v %s" % (tuple(q.shape), tuple(k.shape),
                                                              tuple(v.shape)))
    if o is None:
        o = torch.empty_like(q)
    _need(o, "o", torch.bfloat16, 4)
    if tuple(o.shape) != tuple(q.shape):
        raise ValueError("o must have q's shape")
    if lse is None and want_lse:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    if lse is not None:
        _need(lse, "lse", torch.float32, 3)
        if tuple(lse.shape) != (B, Hq, Sq):
            raise ValueError("lse must be [B,Hq,Sq]")
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, Sq, Skv, d,
            _scale(scale, d), int(bool(causal)))
    if poly is None:
        st = _lib.load().attn_fwd(*args, _stream(stream))
        _check(st, "attn_fwd")
    else:
        st = _lib.load().attn_fwd_exp2_poly(*args, poly, _stream(stream))
        _check(st, "attn_fwd_exp2_poly")
    return o, lse


def attn_fwd_splitkv_workspace_bytes(B, Hq, Sq, Skv, d, causal=False, num_splits=0) -> int:
    return int(_lib.load().attn_fwd_splitkv_workspace_bytes(B, Hq, Sq, Skv, d, int(bool(causal)),
                                                            num_splits))


def attn_fwd_splitkv(q, k, v, o=None, lse=None, scale=None, causal=False, num_splits=0,
                     workspace=None, want_lse=True, stream=None):
    """Prefill with the key range split across workgroups; returns ``(o, lse)``.

    As :func:`attn_fwd`; ``num_splits <= 0`` lets the library choose and
    ``workspace`` (a uint8 GPU tensor of at least
    :func:`attn_fwd_splitkv_workspace_bytes` bytes) is allocated here if
    omitted.
    """
    _need(q, "q", torch.bfloat16, 4)
    _need(k, "k", torch.bfloat16, 4)
    _need(v, "v", torch.bfloat16, 4)
    B, Sq, Hq, d = q.shape
    Skv, Hkv = k.shape[1], k.shape[2]
    if tuple(v.shape) != tuple(k.shape) or k.shape[0] != B or k.shape[3] != d:
        raise ValueError("shape mismatch")
    if o is None:
        o = torch.empty_like(q)
    _need(o, "o", torch.bfloat16, 4)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    if lse is not None:
        _need(lse, "lse", torch.float32, 3)
    nbytes = attn_fwd_splitkv_workspace_bytes(B, Hq, Sq, Skv, d, causal, num_splits)
    if workspace is None and nbytes > 0:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = _lib.load().attn_fwd_splitkv(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv,
                                      Sq, Skv, d, _scale(scale, d), int(bool(causal)),
                                      int(num_splits), _ptr(workspace), ws_bytes,
                                      _stream(stream))
    _check(st, "attn_fwd_splitkv")
    return o, lse


def attn_varlen_check(cu_seqlens_host, total: int) -> int:
    """Validate a host copy of cumulative offsets; returns the longest length."""
    import numpy as np
    cu = np.ascontiguousarray(np.asarray(cu_seqlens_host, dtype=np.int32))
    mx = ctypes.c_int(0)
    st = _lib.load().attn_varlen_check(cu.ctypes.data_as(ctypes.c_void_p), len(cu) - 1,
                                       int(total), ctypes.byref(mx))
    _check(st, "attn_varlen_check")
    return mx.value


def attn_fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, o=None,
                    lse=None, scale=None, causal=False, want_lse=True, stream=None):
    """Attention forward over a packed ragged batch; returns ``(o, lse)``.

    q ``[Tq,Hq,d]``, k/v ``[Tk,Hkv,d]`` bf16; cu_seqlens_* int32 GPU tensors
    of nseq+1 offsets; lse ``[Hq,Tq]`` fp32.
    """
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, torch.bfloat16, 3)
    _need(cu_seqlens_q, "cu_seqlens_q", torch.int32, 1)
    _need(cu_seqlens_k, "cu_seqlens_k", torch.int32, 1)
    Tq, Hq, d = q.shape
    Tk, Hkv = k.shape[0], k.shape[1]
    if tuple(v.shape) != tuple(k.shape) or k.shape[2] != d:
        raise ValueError("shape mismatch")
    nseq = cu_seqlens_q.shape[0] - 1
    if cu_seqlens_k.shape[0] - 1 != nseq:
        raise ValueError("cu_seqlens_q and cu_seqlens_k differ in length")
    if o is None:
        o = torch.empty_like(q)
    _need(o, "o", torch.bfloat16, 3)
    if lse is None and want_lse:
        lse = torch.empty((Hq, Tq), dtype=torch.float32, device=q.device)
    if lse is not None:
        _need(lse, "lse", torch.float32, 2)
        if tuple(lse.shape) != (Hq, Tq):
            raise ValueError("lse must be [Hq,Tq]")
    st = _lib.load().attn_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                     _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), nseq, Tq, Tk,
                                     int(max_seqlen_q), int(max_seqlen_k), Hq, Hkv, d,
                                     _scale(scale, d), int(bool(causal)), _stream(stream))
    _check(st, "attn_fwd_varlen")
    return o, lse


def attn_decode_workspace_bytes(B, Hq, Hkv, Skv, d, num_splits=0) -> int:
    return int(_lib.load().attn_decode_workspace_bytes(B, Hq, Hkv, Skv, d, num_splits))


def attn_decode_varlen_workspace_bytes(B, Hq, Hkv, Skv_max, d) -> int:
    return int(_lib.load().attn_decode_varlen_workspace_bytes(B, Hq, Hkv, Skv_max, d))


def _decode_ws_bytes(B, Hq, Hkv, Skv, d, num_splits, with_lengths):
    # with per-sequence lengths and the library's choice: the workspace of the
    # split by the lengths, so the kernel spreads mixed lengths over the GPU
    if with_lengths and num_splits <= 0:
        return attn_decode_varlen_workspace_bytes(B, Hq, Hkv, Skv, d)
    return attn_decode_workspace_bytes(B, Hq, Hkv, Skv, d, num_splits)


def attn_decode_pick_splits(B, Hq, Hkv, Skv) -> int:
    return int(_lib.load().attn_decode_pick_splits(B, Hq, Hkv, Skv))


def attn_decode(q, k_cache, v_cache, o=None, lse=None, scale=None, num_splits=0, workspace=None,
                want_lse=True, stream=None):
    """Split-KV decode; returns ``(o, lse)``.

    q ``[B,Hq,d]``, caches ``[B,Skv,Hkv,d]`` bf16; o ``[B,Hq,d]`` bf16, lse
    ``[B,Hq]`` fp32.  workspace: a uint8 GPU tensor of at least
    :func:`attn_decode_workspace_bytes` bytes (allocated here if omitted).
    """
    return _decode(q, k_cache, v_cache, None, o, lse, scale, num_splits, workspace, want_lse,
                   stream)


def attn_decode_noalloc(q, k_cache, v_cache, o=None, lse=None, scale=None, num_splits=0,
                        want_lse=True, stream=None):
    """:func:`attn_decode` through the entry point that allocates nothing (its
    split partials live in the library's fixed device scratch); returns
    ``(o, lse)``.  Outputs are allocated here only if not given."""
    _need(q, "q", torch.bfloat16, 3)
    _need(k_cache, "k_cache", torch.bfloat16, 4)
    _need(v_cache, "v_cache", torch.bfloat16, 4)
    B, Hq, d = q.shape
    Skv, Hkv = k_cache.shape[1], k_cache.shape[2]
    if tuple(v_cache.shape) != tuple(k_cache.shape) or k_cache.shape[0] != B or \
            k_cache.shape[3] != d:
        raise ValueError("shape mismatch")
    if o is None:
        o = torch.empty_like(q)
    _need(o, "o", torch.bfloat16, 3)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    if lse is not None:
        _need(lse, "lse", torch.float32, 2)
    st = _lib.load().attn_decode_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(o), _ptr(lse),
                                         B, Hq, Hkv, Skv, d, _scale(scale, d), int(num_splits),
                                         _stream(stream))
    _check(st, "attn_decode_noalloc")
    return o, lse


def attn_decode_varlen(q, k_cache, v_cache, seqlens_k, o=None, lse=None, scale=None,
                       num_splits=0, workspace=None, want_lse=True, stream=None):
    """Decode against caches of per-sequence lengths; returns ``(o, lse)``.

    As :func:`attn_decode`, with ``seqlens_k`` an int32 GPU tensor ``[B]``:
    sequence b attends to its first ``seqlens_k[b]`` cache rows (clamped to
    the cache capacity on the device).  With ``num_splits <= 0`` the
    workspace allocated here (or one of at least
    :func:`attn_decode_varlen_workspace_bytes` bytes) lets the kernel split
    the batch by the lengths themselves.
    """
    _need(seqlens_k, "seqlens_k", torch.int32, 1)
    if seqlens_k.shape[0] != q.shape[0]:
        raise ValueError("seqlens_k must have one entry per sequence")
    return _decode(q, k_cache, v_cache, seqlens_k, o, lse, scale, num_splits, workspace,
                   want_lse, stream)


def attn_decode_paged(q, k_pages, v_pages, block_table, seqlens_k, o=None, lse=None, scale=None,
                      num_splits=0, workspace=None, want_lse=True, stream=None):
    """Decode against a paged KV cache; returns ``(o, lse)``.

    q ``[B,Hq,d]`` bf16; k_pages/v_pages ``[num_pages,page_size,Hkv,d]`` bf16;
    block_table int32 GPU ``[B,max_pages_per_seq]`` (page ids); seqlens_k
    int32 GPU ``[B]``.  Key j of sequence b is row ``j % page_size`` of page
    ``block_table[b, j // page_size]``.
    """
    _need(q, "q", torch.bfloat16, 3)
    _need(k_pages, "k_pages", torch.bfloat16, 4)
    _need(v_pages, "v_pages", torch.bfloat16, 4)
    _need(block_table, "block_table", torch.int32, 2)
    _need(seqlens_k, "seqlens_k", torch.int32, 1)
    B, Hq, d = q.shape
    num_pages, page_size, Hkv = k_pages.shape[0], k_pages.shape[1], k_pages.shape[2]
    if tuple(v_pages.shape) != tuple(k_pages.shape) or k_pages.shape[3] != d:
        raise ValueError("shape mismatch")
    if block_table.shape[0] != B or seqlens_k.shape[0] != B:
        raise ValueError("block_table and seqlens_k must have one row per sequence")
    max_pages = block_table.shape[1]
    if o is None:
        o = torch.empty_like(q)
    _need(o, "o", torch.bfloat16, 3)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    if lse is not None:
        _need(lse, "lse", torch.float32, 2)
    nbytes = _decode_ws_bytes(B, Hq, Hkv, max_pages * page_size, d, num_splits, True)
    if workspace is None and nbytes > 0:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = _lib.load().attn_decode_paged(_ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(o), _ptr(lse),
                                       _ptr(block_table), _ptr(seqlens_k), B, Hq, Hkv, d,
                                       page_size, max_pages, num_pages, _scale(scale, d),
                                       int(num_splits), _ptr(workspace), ws_bytes,
                                       _stream(stream))
    _check(st, "attn_decode_paged")
    return o, lse


def attn_decode_fp8(q, k_cache, v_cache, k_scale, v_scale, seqlens_k=None, o=None, lse=None,
                    scale=None, num_splits=0, workspace=None, want_lse=True, stream=None):
    """Decode against an fp8 (e4m3fn) KV cache; returns ``(o, lse)``.

    q ``[B,Hq,d]`` bf16; k_cache/v_cache ``[B,Skv,Hkv,d]`` of e4m3fn codes
    (``torch.uint8`` or ``torch.float8_e4m3fn``), holding ``k / k_scale`` and
    ``v / v_scale``; seqlens_k an optional int32 GPU ``[B]`` as in
    :func:`attn_decode_varlen`.
    """
    def codes(t, name):
        if isinstance(t, torch.Tensor) and t.dtype == torch.float8_e4m3fn:
            t = t.view(torch.uint8)
        _need(t, name, torch.uint8, 4)
        return t

    _need(q, "q", torch.bfloat16, 3)
    k_cache, v_cache = codes(k_cache, "k_cache"), codes(v_cache, "v_cache")
    B, Hq, d = q.shape
    Skv, Hkv = k_cache.shape[1], k_cache.shape[2]
    if tuple(v_cache.shape) != tuple(k_cache.shape) or k_cache.shape[0] != B or \
            k_cache.shape[3] != d:
        raise ValueError("shape mismatch")
    if seqlens_k is not None:
        _need(seqlens_k, "seqlens_k", torch.int32, 1)
        if seqlens_k.shape[0] != B:
            raise ValueError("seqlens_k must have one entry per sequence")
    if o is None:
        o = torch.empty_like(q)
    _need(o, "o", torch.bfloat16, 3)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    if lse is not None:
        _need(lse, "lse", torch.float32, 2)
    nbytes = _decode_ws_bytes(B, Hq, Hkv, Skv, d, num_splits, seqlens_k is not None)
    if workspace is None and nbytes > 0:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = _lib.load().attn_decode_fp8(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(o), _ptr(lse),
                                     _ptr(seqlens_k), B, Hq, Hkv, Skv, d, _scale(scale, d),
                                     float(k_scale), float(v_scale), int(num_splits),
                                     _ptr(workspace), ws_bytes, _stream(stream))
    _check(st, "attn_decode_fp8")
    return o, lse


def attn_kmeans_assign(x, c, idx=None, dist=None, want_dist=True, stream=None):
    """Nearest centroid of every point; returns ``(idx, dist)``.

    x ``[N,d]`` and c ``[K,d]`` bf16 GPU tensors; idx ``[N]`` int32, dist
    ``[N]`` fp32 (squared distance to the chosen centroid, or None when
    ``want_dist`` is false).
    """
    _need(x, "x", torch.bfloat16, 2)
    _need(c, "c", torch.bfloat16, 2)
    N, d = x.shape
    K = c.shape[0]
    if c.shape[1] != d:
        raise ValueError("x and c must have the same dimension")
    if idx is None:
        idx = torch.empty(N, dtype=torch.int32, device=x.device)
    _need(idx, "idx", torch.int32, 1)
    if dist is None and want_dist:
        dist = torch.empty(N, dtype=torch.float32, device=x.device)
    if dist is not None:
        _need(dist, "dist", torch.float32, 1)
    if idx.shape[0] != N or (dist is not None and dist.shape[0] != N):
        raise ValueError("idx and dist must have one entry per point")
    st = _lib.load().attn_kmeans_assign(_ptr(x), _ptr(c), _ptr(idx), _ptr(dist), N, K, d,
                                        _stream(stream))
    _check(st, "attn_kmeans_assign")
    return idx, dist


def _decode(q, k_cache, v_cache, seqlens_k, o, lse, scale, num_splits, workspace, want_lse,
            stream):
    _need(q, "q", torch.bfloat16, 3)
    _need(k_cache, "k_cache", torch.bfloat16, 4)
    _need(v_cache, "v_cache", torch.bfloat16, 4)
    B, Hq, d = q.shape
    Skv, Hkv = k_cache.shape[1], k_cache.shape[2]
    if tuple(v_cache.shape) != tuple(k_cache.shape) or k_cache.shape[0] != B or \
            k_cache.shape[3] != d:
        raise ValueError("shape mismatch")
    if o is None:
        o = torch.empty_like(q)
    _need(o, "o", torch.bfloat16, 3)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    if lse is not None:
        _need(lse, "lse", torch.float32, 2)
    nbytes = _decode_ws_bytes(B, Hq, Hkv, Skv, d, num_splits, seqlens_k is not None)
    if workspace is None and nbytes > 0:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    lib = _lib.load()
    if seqlens_k is None:
        st = lib.attn_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(o), _ptr(lse), B, Hq,
                             Hkv, Skv, d, _scale(scale, d), int(num_splits), _ptr(workspace),
                             ws_bytes, _stream(stream))
        _check(st, "attn_decode")
    else:
        st = lib.attn_decode_varlen(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(o), _ptr(lse),
                                    _ptr(seqlens_k), B, Hq, Hkv, Skv, d, _scale(scale, d),
                                    int(num_splits), _ptr(workspace), ws_bytes,
                                    _stream(stream))
        _check(st, "attn_decode_varlen")
    return o, lse
