"""Seeded synthetic inputs for the attention workloads.

This module only draws random numbers and rounds them to bfloat16 bit
patterns.  It holds none of the attention arithmetic, so both the CPU oracle
(through the tests) and the GPU path (through the binding) can be fed the very
same bytes from it.

Recipe (one ``numpy.random.default_rng(seed)`` stream per workload):

* prefill / decode: ``standard_normal(shape, float32)`` drawn in the order
  q, k, v; each value is rounded to bfloat16 with round-to-nearest-even.
* long causal prefill: after v, one factor per head ``uniform(0.5, 2.0)``
  (float32) multiplies that head of K in float32 before the single bf16
  rounding, which varies how sharp the softmax is per head.
* fp8 KV cache: q as for decode; K and V drawn as float32 standard normals
  (order q, k, v), each tensor given one scale ``max|x| / 448`` (float32) and
  stored as the FP8 E4M3 ("e4m3fn") codes of ``x / scale`` clipped to
  [-448, 448], rounded to nearest by torch's float8_e4m3fn conversion (a
  per-tensor quantiser of the usual kind; the codes span the format's range).
* k-means assignment: a Gaussian mixture with one component per centroid:
  component means ``mu ~ N(0, 1)`` [K, d], labels ``integers(0, K, N)``,
  points ``x = mu[label] + 0.5 * N(0, 1)`` [N, d] and centroids
  ``c = mu + 0.25 * N(0, 1)`` [K, d] (a k-means state part way through its
  iterations), drawn in that order in float32, each rounded once to bf16.
* ragged batch: the 16 lengths are drawn first with
  ``integers(lo, hi + 1, nseq)`` (inclusive bounds), then q, k, v over the
  packed ``[total, H, d]`` layout.

Arrays are returned as ``uint16`` bit patterns (what the GPU reads) and the
caller can widen them exactly with :func:`bf16_to_f64`.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "f32_to_bf16_bits", "bf16_to_f32", "bf16_to_f64", "WORKLOADS",
    "make_prefill", "make_decode", "make_decode_fp8", "make_varlen", "make_workload",
    "make_kmeans",
]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Inputs are finite normal draws here, so no NaN handling is needed; a NaN
    is rejected rather than silently rounded.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite value in synthetic input")
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 exactly."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float64 exactly."""
    return bf16_to_f32(bits).astype(np.float64)


# The five workloads, with their sizes.  ``scale`` is the float32 value
# 1/sqrt(d) that both sides receive.
WORKLOADS = {
    "tiny": dict(kind="prefill", name="tiny non-causal B1 H2 S256 d64", B=1, Hq=2, Hkv=2,
            Sq=256, Skv=256, d=64, causal=False, seed=1),
    "causal_prefill": dict(kind="prefill", name="causal prefill B4 H16 S2048 d128", B=4, Hq=16, Hkv=16,
            Sq=2048, Skv=2048, d=128, causal=True, seed=2),
    "long_causal": dict(kind="prefill", name="long causal prefill B1 H32 S16384 d128 (K per head x U(0.5,2))",
            B=1, Hq=32, Hkv=32, Sq=16384, Skv=16384, d=128, causal=True, seed=3,
            k_head_scale=True),
    "gqa_decode": dict(kind="decode", name="GQA decode B64 Hq32 Hkv8 Skv4096 d128 8 splits", B=64, Hq=32,
            Hkv=8, Skv=4096, d=128, num_splits=8, seed=4),
    "ragged": dict(kind="varlen", name="ragged causal 16 seqs L~U[128,8192] H32 d128", nseq=16,
            lo=128, hi=8192, H=32, d=128, causal=True, seed=5),
}


def default_scale(d: int) -> float:
    """1/sqrt(d) rounded to float32 (the value handed to the kernel)."""
    return float(np.float32(1.0) / np.sqrt(np.float32(d)))


def make_prefill(seed, B, Hq, Hkv, Sq, Skv, d, k_head_scale=False):
    """q [B,Sq,Hq,d], k/v [B,Skv,Hkv,d] as bf16 bit patterns."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Sq, Hq, d), dtype=np.float32)
    k = rng.standard_normal((B, Skv, Hkv, d), dtype=np.float32)
    v = rng.standard_normal((B, Skv, Hkv, d), dtype=np.float32)
    out = {}
    if k_head_scale:
        c = rng.uniform(0.5, 2.0, size=Hkv).astype(np.float32)
        k = k * c[None, None, :, None]
        out["k_head_scale"] = c
    out.update(q=f32_to_bf16_bits(q), k=f32_to_bf16_bits(k), v=f32_to_bf16_bits(v))
    return out


def make_decode(seed, B, Hq, Hkv, Skv, d):
    """q [B,Hq,d], k/v cache [B,Skv,Hkv,d] as bf16 bit patterns."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, d), dtype=np.float32)
    k = rng.standard_normal((B, Skv, Hkv, d), dtype=np.float32)
    v = rng.standard_normal((B, Skv, Hkv, d), dtype=np.float32)
    return dict(q=f32_to_bf16_bits(q), k=f32_to_bf16_bits(k), v=f32_to_bf16_bits(v))


def make_decode_fp8(seed, B, Hq, Hkv, Skv, d):
    """q [B,Hq,d] (bf16 bits); k/v caches [B,Skv,Hkv,d] as uint8 e4m3fn
    codes with float32 per-tensor scales ``k_scale`` and ``v_scale``."""
    import torch
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, d), dtype=np.float32)
    out = dict(q=f32_to_bf16_bits(q))
    for name in ("k", "v"):
        x = rng.standard_normal((B, Skv, Hkv, d), dtype=np.float32)
        sc = np.float32(np.abs(x).max() / np.float32(448.0))
        y = np.clip(x / sc, np.float32(-448.0), np.float32(448.0)).astype(np.float32)
        codes = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        out[name] = codes
        out[name + "_scale"] = float(sc)
    return out


def make_kmeans(seed, N, K, d):
    """Points x [N,d] and centroids c [K,d] as bf16 bit patterns (mixture recipe above)."""
    rng = np.random.default_rng(seed)
    mu = rng.standard_normal((K, d), dtype=np.float32)
    label = rng.integers(0, K, N)
    x = mu[label] + np.float32(0.5) * rng.standard_normal((N, d), dtype=np.float32)
    c = mu + np.float32(0.25) * rng.standard_normal((K, d), dtype=np.float32)
    return dict(x=f32_to_bf16_bits(x), c=f32_to_bf16_bits(c), label=label)


def make_paged(seed, B, Hq, Hkv, d, page_size, max_pages, num_pages):
    """A paged KV cache: q [B,Hq,d], k/v pages [num_pages,page_size,Hkv,d]
    (bf16 bit patterns) and an int32 block table [B,max_pages] of distinct
    page ids in random order (needs num_pages >= B*max_pages).  ``gather``
    turns it back into a dense [B, max_pages*page_size, Hkv, d] cache.
    """
    if num_pages < B * max_pages:
        raise ValueError("the pool must hold every table entry")
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, d), dtype=np.float32)
    k = rng.standard_normal((num_pages, page_size, Hkv, d), dtype=np.float32)
    v = rng.standard_normal((num_pages, page_size, Hkv, d), dtype=np.float32)
    table = rng.permutation(num_pages)[:B * max_pages].reshape(B, max_pages).astype(np.int32)
    return dict(q=f32_to_bf16_bits(q), k_pages=f32_to_bf16_bits(k),
                v_pages=f32_to_bf16_bits(v), block_table=table)


def gather_pages(pages, table):
    """Dense [B, max_pages*page_size, H, d] view of paged storage (indexing only)."""
    B, max_pages = table.shape
    out = pages[table.reshape(-1)]                       # [B*max_pages, page, H, d]
    return out.reshape(B, max_pages * pages.shape[1], pages.shape[2], pages.shape[3])


def make_varlen(seed, nseq, lo, hi, H, d, Hkv=None, lengths=None):
    """Packed ragged batch: q/k/v [total,H,d] and int32 cu_seqlens [nseq+1].

    Self-attention lengths (the same for q and k).  ``lengths`` overrides the
    draw (used by small tests); the rng still starts from ``seed``.
    """
    Hkv = H if Hkv is None else Hkv
    rng = np.random.default_rng(seed)
    if lengths is None:
        lengths = rng.integers(lo, hi + 1, nseq)
    lengths = np.asarray(lengths, dtype=np.int64)
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)
    total = int(cu[-1])
    q = rng.standard_normal((total, H, d), dtype=np.float32)
    k = rng.standard_normal((total, Hkv, d), dtype=np.float32)
    v = rng.standard_normal((total, Hkv, d), dtype=np.float32)
    return dict(q=f32_to_bf16_bits(q), k=f32_to_bf16_bits(k), v=f32_to_bf16_bits(v),
                cu_seqlens=cu, lengths=lengths)


def make_varlen_cross(seed, lengths_q, lengths_k, H, d, Hkv=None):
    """Packed ragged batch whose query and key lengths differ per sequence.

    The shape of chunked prefill: sequence s brings ``lengths_q[s]`` new
    query rows and attends to ``lengths_k[s]`` keys (its earlier tokens and
    the new ones).  Either length may be 0.  q is [total_q,H,d], k/v are
    [total_k,Hkv,d], and cu_seqlens_q / cu_seqlens_k are int32 [nseq+1].
    """
    Hkv = H if Hkv is None else Hkv
    lq = np.asarray(lengths_q, dtype=np.int64)
    lk = np.asarray(lengths_k, dtype=np.int64)
    if lq.shape != lk.shape:
        raise ValueError("lengths_q and lengths_k must have one entry per sequence")
    rng = np.random.default_rng(seed)
    cu_q = np.zeros(len(lq) + 1, dtype=np.int32)
    cu_k = np.zeros(len(lk) + 1, dtype=np.int32)
    cu_q[1:] = np.cumsum(lq)
    cu_k[1:] = np.cumsum(lk)
    q = rng.standard_normal((int(cu_q[-1]), H, d), dtype=np.float32)
    k = rng.standard_normal((int(cu_k[-1]), Hkv, d), dtype=np.float32)
    v = rng.standard_normal((int(cu_k[-1]), Hkv, d), dtype=np.float32)
    return dict(q=f32_to_bf16_bits(q), k=f32_to_bf16_bits(k), v=f32_to_bf16_bits(v),
                cu_seqlens_q=cu_q, cu_seqlens_k=cu_k, lengths_q=lq, lengths_k=lk)


def make_workload(name: str):
    """Inputs and the spec for one of the five named workloads."""
    spec = dict(WORKLOADS[name])
    if spec["kind"] == "prefill":
        data = make_prefill(spec["seed"], spec["B"], spec["Hq"], spec["Hkv"], spec["Sq"],
                            spec["Skv"], spec["d"], spec.get("k_head_scale", False))
    elif spec["kind"] == "decode":
        data = make_decode(spec["seed"], spec["B"], spec["Hq"], spec["Hkv"], spec["Skv"],
                           spec["d"])
    else:
        data = make_varlen(spec["seed"], spec["nseq"], spec["lo"], spec["hi"], spec["H"],
                           spec["d"])
    spec["scale"] = default_scale(spec["d"])
    return spec, data
