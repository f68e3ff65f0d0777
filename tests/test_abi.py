"""The C ABI on a host with no GPU: every declared symbol is exported, and
invalid arguments are rejected on the host before any launch.

Only argument combinations that FAIL validation are passed here (fake device
pointers are never launched on), so no HIP call is made.
"""
import ctypes
import os
import re

import pytest

import tiled_attention_transformer_amd as pkg
from tiled_attention_transformer_amd import _lib


def _gpu_visible() -> bool:
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return False


# The fake device addresses below must never reach a kernel: on a machine
# with a GPU a validation regression would launch on them, so these host
# tests run only where no GPU is visible.
pytestmark = pytest.mark.skipif(_gpu_visible(), reason="host-only ABI tests (fake device pointers)")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")

OK, NULLPTR, SHAPE, BAD_D, GQA, ALIGN, WS, SEQ, HIP, SCALE, SCRATCH, OPTION = range(12)
P = 1 << 20          # a 16-byte aligned fake address (never dereferenced)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return pkg.load()


def test_library_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) == 16, names
    raw = ctypes.CDLL(_lib.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), n
    assert set(names) == set(_lib.SIGNATURES)


def test_status_strings(lib):
    for s in range(12):
        text = lib.attn_status_string(s)
        assert text and text != b"unknown status"
    assert lib.attn_status_string(99) == b"unknown status"


def fwd(lib, q=P, k=P, v=P, o=P, lse=None, B=1, Hq=2, Hkv=2, Sq=8, Skv=8, d=128, scale=0.1,
        causal=0):
    return lib.attn_fwd(q, k, v, o, lse, B, Hq, Hkv, Sq, Skv, d, scale, causal, None)


def test_fwd_validation(lib):
    assert fwd(lib, q=None) == NULLPTR
    assert fwd(lib, o=None) == NULLPTR
    assert fwd(lib, B=0) == SHAPE
    assert fwd(lib, Sq=-1) == SHAPE
    assert fwd(lib, Skv=0) == SHAPE
    assert fwd(lib, Sq=1 << 30, B=1 << 10) == SHAPE
    assert fwd(lib, d=96) == BAD_D
    assert fwd(lib, d=256) == BAD_D
    assert fwd(lib, Hq=6, Hkv=4) == GQA
    assert fwd(lib, scale=0.0) == SCALE
    assert fwd(lib, scale=-1.0) == SCALE
    assert fwd(lib, scale=float("nan")) == SCALE
    assert fwd(lib, scale=float("inf")) == SCALE
    assert fwd(lib, q=P + 8) == ALIGN
    assert fwd(lib, v=P + 2) == ALIGN
    assert fwd(lib, lse=P + 2) == ALIGN
    # the first failing rule wins, in a fixed order
    assert fwd(lib, q=None, d=96) == NULLPTR
    assert fwd(lib, d=96, Hq=3, Hkv=2) == BAD_D


def fwd_poly(lib, poly, q=P, B=1, d=128, scale=0.1):
    return lib.attn_fwd_exp2_poly(q, P, P, P, None, B, 2, 2, 8, 8, d, scale, 1, poly, None)


def test_fwd_exp2_poly_validation(lib):
    # only the documented shares are accepted; the size checks come first
    for bad in (-1, 1, 2, 3, 5, 12, 32, 64):
        assert fwd_poly(lib, bad) == OPTION, bad
    assert fwd_poly(lib, 8, q=None) == NULLPTR
    assert fwd_poly(lib, 7, B=0) == SHAPE
    assert fwd_poly(lib, 8, d=96) == BAD_D
    assert fwd_poly(lib, 4, scale=0.0) == SCALE
    assert fwd_poly(lib, 16, q=P + 8) == ALIGN


def varlen(lib, cu_q=P, cu_k=P, nseq=2, tq=10, tk=10, mq=6, mk=6, Hq=2, Hkv=1, d=64,
           scale=0.1, q=P):
    return lib.attn_fwd_varlen(q, P, P, P, None, cu_q, cu_k, nseq, tq, tk, mq, mk, Hq, Hkv, d,
                               scale, 1, None)


def test_varlen_validation(lib):
    assert varlen(lib, cu_q=None) == NULLPTR
    assert varlen(lib, q=None) == NULLPTR
    assert varlen(lib, nseq=0) == SHAPE
    assert varlen(lib, tq=0) == SHAPE
    assert varlen(lib, mq=11) == SEQ          # longer than the whole batch
    assert varlen(lib, d=32) == BAD_D
    assert varlen(lib, Hq=3, Hkv=2) == GQA
    assert varlen(lib, scale=0.0) == SCALE
    assert varlen(lib, cu_q=P + 2) == ALIGN


def check(lib, cu, total):
    import numpy as np
    a = np.asarray(cu, dtype=np.int32)
    mx = ctypes.c_int(-1)
    st = lib.attn_varlen_check(a.ctypes.data_as(ctypes.c_void_p), len(a) - 1, total,
                               ctypes.byref(mx))
    return st, mx.value


def test_varlen_check(lib):
    assert check(lib, [0, 3, 3, 10], 10) == (OK, 7)
    assert check(lib, [0, 5], 5) == (OK, 5)
    assert check(lib, [1, 3, 10], 10)[0] == SEQ      # does not start at 0
    assert check(lib, [0, 3, 2, 10], 10)[0] == SEQ   # decreasing
    assert check(lib, [0, 3, 9], 10)[0] == SEQ       # does not end at total
    assert check(lib, [0], 0)[0] == SEQ              # no sequence
    assert lib.attn_varlen_check(None, 1, 1, None) == NULLPTR


def decode(lib, B=2, Hq=8, Hkv=2, Skv=100, d=128, scale=0.1, splits=4, ws=P, wsb=1 << 30,
           q=P, o=P):
    return lib.attn_decode(q, P, P, o, None, B, Hq, Hkv, Skv, d, scale, splits, ws, wsb, None)


def test_decode_validation(lib):
    assert decode(lib, q=None) == NULLPTR
    assert decode(lib, B=0) == SHAPE
    assert decode(lib, Skv=0) == SHAPE
    assert decode(lib, d=80) == BAD_D
    assert decode(lib, Hq=6, Hkv=4) == GQA
    assert decode(lib, scale=float("nan")) == SCALE
    assert decode(lib, o=P + 4) == ALIGN
    need = lib.attn_decode_workspace_bytes(2, 8, 2, 100, 128, 4)
    assert need == 4 * 2 * 8 * (128 + 1) * 4
    assert decode(lib, ws=None) == WS
    assert decode(lib, wsb=need - 1) == WS
    assert decode(lib, ws=P + 4, wsb=need) == ALIGN
    assert lib.attn_decode_workspace_bytes(2, 8, 2, 100, 128, 1) == 0
    assert lib.attn_decode_workspace_bytes(2, 8, 3, 100, 128, 4) == 0    # bad ratio
    assert lib.attn_decode_workspace_bytes(2, 8, 2, 100, 96, 4) == 0     # bad d


def decode_varlen(lib, seqlens=P, B=2, Hq=8, Hkv=2, Skv=100, d=128, scale=0.1, splits=4, ws=P,
                  wsb=1 << 30, q=P):
    return lib.attn_decode_varlen(q, P, P, P, None, seqlens, B, Hq, Hkv, Skv, d, scale, splits,
                                  ws, wsb, None)


def test_decode_varlen_validation(lib):
    assert decode_varlen(lib, seqlens=None) == NULLPTR
    assert decode_varlen(lib, seqlens=P + 2) == ALIGN
    assert decode_varlen(lib, q=None) == NULLPTR
    assert decode_varlen(lib, Skv=0) == SHAPE
    assert decode_varlen(lib, d=96) == BAD_D
    assert decode_varlen(lib, Hq=6, Hkv=4) == GQA
    assert decode_varlen(lib, scale=0.0) == SCALE
    assert decode_varlen(lib, ws=None) == WS


def decode_paged(lib, table=P, seqlens=P, B=2, Hq=8, Hkv=2, d=128, page=16, maxp=8, npages=32,
                 scale=0.1, splits=4, ws=P, wsb=1 << 30, q=P):
    return lib.attn_decode_paged(q, P, P, P, None, table, seqlens, B, Hq, Hkv, d, page, maxp,
                                 npages, scale, splits, ws, wsb, None)


def test_decode_paged_validation(lib):
    assert decode_paged(lib, table=None) == NULLPTR
    assert decode_paged(lib, seqlens=None) == NULLPTR
    assert decode_paged(lib, q=None) == NULLPTR
    assert decode_paged(lib, table=P + 2) == ALIGN
    assert decode_paged(lib, seqlens=P + 1) == ALIGN
    for page in (0, 8, 24, -16):                 # not a positive multiple of 16
        assert decode_paged(lib, page=page) == SHAPE
    assert decode_paged(lib, maxp=0) == SHAPE
    assert decode_paged(lib, npages=0) == SHAPE
    assert decode_paged(lib, d=96) == BAD_D
    assert decode_paged(lib, Hq=6, Hkv=4) == GQA
    assert decode_paged(lib, scale=float("inf")) == SCALE
    assert decode_paged(lib, ws=None) == WS


def decode_fp8(lib, seqlens=None, B=2, Hq=8, Hkv=2, Skv=64, d=128, scale=0.1, ks=0.01, vs=0.01,
               splits=4, ws=P, wsb=1 << 30, q=P, k=P, v=P):
    return lib.attn_decode_fp8(q, k, v, P, None, seqlens, B, Hq, Hkv, Skv, d, scale, ks, vs,
                               splits, ws, wsb, None)


def test_decode_fp8_validation(lib):
    assert decode_fp8(lib, q=None) == NULLPTR
    assert decode_fp8(lib, k=None) == NULLPTR
    assert decode_fp8(lib, v=None) == NULLPTR
    assert decode_fp8(lib, k=P + 8) == ALIGN
    assert decode_fp8(lib, seqlens=P + 2) == ALIGN
    assert decode_fp8(lib, Skv=0) == SHAPE
    assert decode_fp8(lib, d=96) == BAD_D
    assert decode_fp8(lib, Hq=6, Hkv=4) == GQA
    assert decode_fp8(lib, scale=0.0) == SCALE
    for bad in (0.0, -1.0, float("inf"), float("nan")):
        assert decode_fp8(lib, ks=bad) == SCALE
        assert decode_fp8(lib, vs=bad) == SCALE
    assert decode_fp8(lib, scale=1e-30, ks=1e-30) == SCALE    # product underflows to 0
    assert decode_fp8(lib, ws=None) == WS
    assert decode_fp8(lib, wsb=16) == WS


def kmeans(lib, x=P, c=P, idx=P, dist=P, N=1000, K=64, d=128):
    return lib.attn_kmeans_assign(x, c, idx, dist, N, K, d, None)


def test_kmeans_assign_validation(lib):
    assert kmeans(lib, x=None) == NULLPTR
    assert kmeans(lib, c=None) == NULLPTR
    assert kmeans(lib, idx=None) == NULLPTR
    assert kmeans(lib, N=0) == SHAPE
    assert kmeans(lib, K=-1) == SHAPE
    assert kmeans(lib, d=96) == BAD_D
    assert kmeans(lib, d=256) == BAD_D
    assert kmeans(lib, x=P + 8) == ALIGN
    assert kmeans(lib, c=P + 4) == ALIGN
    assert kmeans(lib, idx=P + 2) == ALIGN
    assert kmeans(lib, dist=P + 1) == ALIGN


def fwd_split(lib, q=P, o=P, B=1, Hq=32, Hkv=8, Sq=512, Skv=8192, d=128, scale=0.1, causal=1,
              splits=4, ws=P, wsb=1 << 30):
    return lib.attn_fwd_splitkv(q, P, P, o, None, B, Hq, Hkv, Sq, Skv, d, scale, causal, splits,
                                ws, wsb, None)


def test_fwd_splitkv_validation(lib):
    assert fwd_split(lib, q=None) == NULLPTR
    assert fwd_split(lib, o=None) == NULLPTR
    assert fwd_split(lib, Sq=0) == SHAPE
    assert fwd_split(lib, d=96) == BAD_D
    assert fwd_split(lib, Hq=6, Hkv=4) == GQA
    assert fwd_split(lib, scale=float("nan")) == SCALE
    assert fwd_split(lib, q=P + 2) == ALIGN
    assert fwd_split(lib, ws=None) == WS
    need = lib.attn_fwd_splitkv_workspace_bytes(1, 32, 512, 8192, 128, 1, 4)
    assert need == 4 * 32 * 512 * 129 * 4
    assert fwd_split(lib, wsb=need - 4) == WS
    assert fwd_split(lib, ws=P + 8) == ALIGN
    assert fwd_split(lib, splits=2000) == SHAPE
    ws = lambda *a: lib.attn_fwd_splitkv_workspace_bytes(*a)
    # library's choice: ~one item per CU (256), shares averaging >= 1024 keys
    assert ws(1, 32, 256, 8192, 128, 1, 0) == 7 * 32 * 256 * 129 * 4     # 32 items; 8064 keys
    assert ws(1, 32, 256, 16384, 128, 1, 0) == 8 * 32 * 256 * 129 * 4    # 32 items x 8
    assert ws(1, 32, 512, 8192, 128, 1, 0) == 4 * 32 * 512 * 129 * 4     # 64 items x 4
    assert ws(1, 8, 4096, 4096, 128, 1, 0) == 2 * 8 * 4096 * 129 * 4     # 128 items; 2048 keys
    assert ws(1, 32, 1024, 1024, 128, 1, 0) == 0       # causal: 512 keys per row on average
    assert ws(1, 32, 1024, 1024, 128, 0, 0) == 0       # full rows: 1024 keys, one share
    assert ws(4, 16, 2048, 2048, 128, 1, 0) == 0       # 512 items: no split
    assert ws(1, 32, 512, 8192, 128, 1, 1) == 0
    assert ws(0, 32, 512, 8192, 128, 1, 4) == 0


def test_decode_split_choice(lib):
    # about one work item per compute unit (256), chunks of at least 512 keys
    assert lib.attn_decode_pick_splits(64, 32, 8, 4096) == 1      # 512 groups already
    assert lib.attn_decode_pick_splits(4, 32, 8, 16384) == 8      # 32 groups x 8
    assert lib.attn_decode_pick_splits(1, 32, 8, 32768) == 32     # 8 groups x 32
    assert lib.attn_decode_pick_splits(1, 32, 8, 4096) == 8       # capped: 512-key chunks
    assert lib.attn_decode_pick_splits(1, 64, 1, 100000) == 128   # two column blocks x 128
    assert lib.attn_decode_pick_splits(1, 8, 1, 100000) == 196    # one group: capped by length
    assert lib.attn_decode_pick_splits(1, 1, 1, 100) == 1
    assert lib.attn_decode_pick_splits(1, 3, 2, 100) == 0
    # balance: 384 groups are 1.5 items per workgroup (a half-empty second
    # round); two chunks give 768, three full rounds
    assert lib.attn_decode_pick_splits(48, 32, 8, 4096) == 2
    assert lib.attn_decode_pick_splits(20, 32, 8, 4096) == 3        # 160 groups: 480 items
    assert lib.attn_decode_pick_splits(96, 32, 8, 4096) == 1        # 768 groups: full rounds
    assert lib.attn_decode_pick_splits(40, 32, 8, 8192) == 3        # 320 groups: 960 items
    auto = lib.attn_decode_workspace_bytes(1, 32, 8, 4096, 128, 0)
    assert auto == lib.attn_decode_workspace_bytes(1, 32, 8, 4096, 128, 8)


def test_decode_workspace_of_the_gqa_decode_workload(lib):
    """B64 Hq32 Hkv8 Skv4096 d128: the library's choice is whole sequences
    (512 groups fill the GPU) and needs no workspace; an explicit 8 chunks
    is honoured and needs the partials (8 x 64 x 32 x (128 + 1) fp32)."""
    assert lib.attn_decode_pick_splits(64, 32, 8, 4096) == 1
    assert lib.attn_decode_workspace_bytes(64, 32, 8, 4096, 128, 0) == 0
    assert lib.attn_decode_workspace_bytes(64, 32, 8, 4096, 128, 1) == 0
    assert lib.attn_decode_workspace_bytes(64, 32, 8, 4096, 128, 8) == 8 * 64 * 32 * 129 * 4
    # 8 chunks without a workspace are refused before any launch
    assert lib.attn_decode(P, P, P, P, None, 64, 32, 8, 4096, 128, 0.088, 8, None, 0,
                           None) == WS


def test_decode_varlen_workspace_bytes(lib):
    """The split by the lengths: a header (16 bytes, then one int per sequence
    and one more, padded to 16 bytes), then fp32 partials with their
    log-sum-exp (d + 1 values) in a row per (sequence, query head) and
    min(Hq / Hkv, 32) rows per wave of the 1024-wave grid; past 2048
    sequences the capacity split's size."""
    vw = lib.attn_decode_varlen_workspace_bytes
    hdr = lambda B: 16 + -(-4 * (B + 1) // 16) * 16
    assert vw(64, 32, 8, 32768, 128) == hdr(64) + (64 * 32 + 1024 * 4) * 129 * 4
    assert vw(2, 8, 2, 1000, 64) == hdr(2) + (2 * 8 + 1024 * 4) * 65 * 4
    assert vw(1, 64, 1, 300, 128) == hdr(1) + (64 + 1024 * 32) * 129 * 4   # two blocks of 32
    assert vw(3, 6, 2, 5, 128) == hdr(3) + (18 + 1024 * 3) * 129 * 4
    assert vw(2049, 8, 8, 4096, 128) == lib.attn_decode_workspace_bytes(2049, 8, 8, 4096, 128, 0)
    assert vw(2048, 8, 8, 4096, 128) == hdr(2048) + (2048 * 8 + 1024) * 129 * 4
    # tile positions past an int: the capacity split
    big = 0x7fffffff // 32
    assert vw(2048, 8, 1, big, 64) == lib.attn_decode_workspace_bytes(2048, 8, 1, big, 64, 0)
    assert vw(2, 8, 3, 100, 128) == 0      # bad ratio
    assert vw(2, 8, 2, 100, 96) == 0       # bad d
    assert vw(0, 8, 2, 100, 128) == 0      # no sequences


def test_decode_noalloc_validation(lib):
    """The no-allocation decode: attn_decode's checks in the same order, and
    sizes whose split partials exceed the fixed 16 MiB scratch refused before
    any launch (and before the scratch is looked up)."""
    def nd(q=P, o=P, lse=None, B=2, Hq=8, Hkv=2, Skv=100, d=128, scale=0.1, splits=4):
        return lib.attn_decode_noalloc(q, P, P, o, lse, B, Hq, Hkv, Skv, d, scale, splits, None)
    assert nd(q=None) == NULLPTR
    assert nd(B=0) == SHAPE
    assert nd(d=80) == BAD_D
    assert nd(Hq=6, Hkv=4) == GQA
    assert nd(scale=float("inf")) == SCALE
    assert nd(splits=70000) == SHAPE
    assert nd(o=P + 4) == ALIGN
    assert nd(lse=P + 2) == ALIGN
    # B64 Hq32 Hkv8 d128: 8 chunks of partials take 8.45 MB, 16 chunks 16.9 MB
    assert lib.attn_decode_workspace_bytes(64, 32, 8, 4096, 128, 16) > 16 << 20
    assert nd(B=64, Hq=32, Hkv=8, Skv=4096, splits=16) == SCRATCH
    assert nd(B=1024, Hq=64, Hkv=8, Skv=4096, splits=2) == SCRATCH
