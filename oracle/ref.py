"""Plain fp64 attention oracle (numpy).  TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may use
this module; the library never calls it.

Sources (cited by page title and section):

* lecompute.fr, "FlashAttention-4 : limites du calcul matriciel", section
  "Entre deux multiplications il faut fabriquer les poids": queries are
  compared with keys by a first matrix product giving scores; a softmax turns
  the scores into positive weights that sum to one; a second product uses the
  weights to mix the values.  Tiling (same section) computes the same result
  without storing the score matrix, so the plain definition below is the
  reference for the tiled kernels.
* same page, section "Déplacer une partie des exponentielles": the tiled
  softmax keeps one common scale for the old and the new contributions, and a
  value that has overflowed cannot be repaired by the final normalisation.
  :func:`attention_tiled` follows that description step by step.
* same page, section "Le FP4 ajoute un compromis numérique": a non-causal
  forward may use every position; under the causal mask a position sees only
  the positions it is allowed to.

Readings where the pages are silent (each is listed in the design notes):

* causal alignment when ``Sq != Skv`` is bottom-right: query ``i`` may see key
  ``j`` iff ``j <= i + (Skv - Sq)``;
* a row with no allowed key gives ``O = 0`` and ``LSE = -inf``;
* LSE is the natural log of the sum of ``exp(scale * q.k)`` over the allowed
  keys;
* GQA groups consecutive query heads: query head ``h`` reads KV head
  ``h // (Hq // Hkv)``;
* layouts: q/o ``[B,S,Hq,d]``, k/v ``[B,S,Hkv,d]``, lse ``[B,Hq,Sq]``; packed
  ragged batches use ``[total,H,d]`` with int32 cumulative offsets.

All arithmetic is float64 on the exact (already bf16-rounded) input values.
Matrix products are numpy's; there is no blocking, fusion or reordering other
than what :func:`attention_tiled` and :func:`decode_split` state on purpose.
"""
from __future__ import annotations

import numpy as np

NEG_INF = -np.inf


def allowed_mask(Sq: int, Skv: int, causal: bool) -> np.ndarray:
    """Boolean ``[Sq, Skv]``: may query ``i`` attend to key ``j``.

    Non-causal: every key.  Causal: ``j <= i + (Skv - Sq)`` (bottom-right
    alignment; equals the plain lower triangle when ``Sq == Skv``).
    """
    if not causal:
        return np.ones((Sq, Skv), dtype=bool)
    i = np.arange(Sq)[:, None]
    j = np.arange(Skv)[None, :]
    return j <= i + (Skv - Sq)


def softmax_rows(s: np.ndarray, allowed: np.ndarray):
    """Row softmax over the allowed entries of a score matrix.

    Returns ``(p, m, l)``: weights ``p`` (0 where not allowed), the row
    maximum ``m`` and the row sum ``l = sum_j exp(s_ij - m_i)``.  Subtracting
    the row maximum keeps every exponent <= 0, so nothing overflows.  A row
    with no allowed entry gets ``p = 0``, ``m = -inf``, ``l = 0``.
    """
    s = np.where(allowed, s, NEG_INF)
    m = s.max(axis=-1, initial=NEG_INF)         # also defined for zero keys
    any_ok = allowed.any(axis=-1)
    m_safe = np.where(any_ok, m, 0.0)
    e = np.where(allowed, np.exp(s - m_safe[..., None]), 0.0)
    l = e.sum(axis=-1)
    p = np.where(any_ok[..., None], e / np.where(l > 0, l, 1.0)[..., None], 0.0)
    return p, np.where(any_ok, m, NEG_INF), l


def _head_attention(q, k, v, scale, causal):
    """One (batch, head): q ``[Sq,d]``, k/v ``[Skv,d]`` -> o ``[Sq,d]``, lse ``[Sq]``."""
    Sq, Skv = q.shape[0], k.shape[0]
    s = scale * (q @ k.T)                       # first product: scores
    ok = allowed_mask(Sq, Skv, causal)
    p, m, l = softmax_rows(s, ok)               # weights, rows sum to one
    o = p @ v                                   # second product mixes V
    with np.errstate(divide="ignore"):
        lse = np.where(l > 0, m + np.log(np.where(l > 0, l, 1.0)), NEG_INF)
    return o, lse


def _check_prefill_shapes(q, k, v):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("expected [B,S,H,d] arrays")
    B, Sq, Hq, d = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[3] != d:
        raise ValueError("k/v shape mismatch")
    Hkv = k.shape[2]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    return B, Sq, Hq, Hkv, k.shape[1], d


def attention(q, k, v, scale, causal=False):
    """Full attention forward, the plain definition.

    q ``[B,Sq,Hq,d]``, k/v ``[B,Skv,Hkv,d]`` (float64) -> o ``[B,Sq,Hq,d]``,
    lse ``[B,Hq,Sq]``.  Materialises every masked score row.
    """
    B, Sq, Hq, Hkv, Skv, d = _check_prefill_shapes(q, k, v)
    g = Hq // Hkv
    o = np.zeros((B, Sq, Hq, d))
    lse = np.zeros((B, Hq, Sq))
    for b in range(B):
        for h in range(Hq):
            hk = h // g
            o[b, :, h, :], lse[b, h, :] = _head_attention(
                q[b, :, h, :], k[b, :, hk, :], v[b, :, hk, :], scale, causal)
    return o, lse


def attention_probs(q, k, scale, causal=False):
    """The softmax weights ``[B,Hq,Sq,Skv]`` (for the invariant checks)."""
    B, Sq, Hq, d = q.shape
    Hkv, Skv = k.shape[2], k.shape[1]
    g = Hq // Hkv
    out = np.zeros((B, Hq, Sq, Skv))
    ok = allowed_mask(Sq, Skv, causal)
    for b in range(B):
        for h in range(Hq):
            s = scale * (q[b, :, h, :] @ k[b, :, h // g, :].T)
            out[b, h] = softmax_rows(s, ok)[0]
    return out


def attention_tiled(q, k, v, scale, causal=False, br=64, bc=64):
    """Tile-by-tile attention with an online softmax, in float64.

    Follows the FlashAttention-4 page: the work is cut into blocks of ``br``
    query rows and ``bc`` keys; each key block updates a running row maximum
    ``m`` (the common scale), a running sum ``l`` and an output accumulator,
    so no full score row is ever held.  When the maximum grows, the previous
    sum and accumulator are multiplied by ``exp(m_old - m_new)`` to bring them
    onto the new scale; the output is divided by ``l`` once at the end.  A
    block in which a row has no allowed key leaves that row unchanged (its
    scale stays ``-inf`` and ``exp(-inf - (-inf))`` is never formed).
    """
    B, Sq, Hq, Hkv, Skv, d = _check_prefill_shapes(q, k, v)
    g = Hq // Hkv
    ok_all = allowed_mask(Sq, Skv, causal)
    o = np.zeros((B, Sq, Hq, d))
    lse = np.zeros((B, Hq, Sq))
    for b in range(B):
        for h in range(Hq):
            hk = h // g
            for r0 in range(0, Sq, br):
                r1 = min(Sq, r0 + br)
                qt = q[b, r0:r1, h, :]
                m = np.full(r1 - r0, NEG_INF)
                l = np.zeros(r1 - r0)
                acc = np.zeros((r1 - r0, d))
                for c0 in range(0, Skv, bc):
                    c1 = min(Skv, c0 + bc)
                    ok = ok_all[r0:r1, c0:c1]
                    s = np.where(ok, scale * (qt @ k[b, c0:c1, hk, :].T), NEG_INF)
                    m_new = np.maximum(m, s.max(axis=1))
                    live = m_new > NEG_INF          # rows with an allowed key so far
                    m_ref = np.where(live, m_new, 0.0)
                    alpha = np.where(live, np.exp(m - m_ref), 1.0)
                    p = np.where(ok, np.exp(s - m_ref[:, None]), 0.0)
                    l = alpha * l + p.sum(axis=1)
                    acc = alpha[:, None] * acc + p @ v[b, c0:c1, hk, :]
                    m = m_new
                with np.errstate(divide="ignore", invalid="ignore"):
                    o[b, r0:r1, h, :] = np.where(l[:, None] > 0,
                                                 acc / np.where(l > 0, l, 1.0)[:, None], 0.0)
                    lse[b, h, r0:r1] = np.where(l > 0, m + np.log(np.where(l > 0, l, 1.0)),
                                                NEG_INF)
    return o, lse


def attention_varlen(q, k, v, cu_q, cu_k, scale, causal=False):
    """Packed ragged batch: q ``[Tq,Hq,d]``, k/v ``[Tk,Hkv,d]``.

    Sequence ``s`` owns query rows ``cu_q[s]:cu_q[s+1]`` and keys
    ``cu_k[s]:cu_k[s+1]``; no key of another sequence is ever seen, and the
    causal mask is applied inside each sequence.  lse is ``[Hq, Tq]``.
    """
    Tq, Hq, d = q.shape
    o = np.zeros((Tq, Hq, d))
    lse = np.zeros((Hq, Tq))
    for s in range(len(cu_q) - 1):
        a, b_ = int(cu_q[s]), int(cu_q[s + 1])
        c, e = int(cu_k[s]), int(cu_k[s + 1])
        if b_ == a:
            continue
        os_, ls_ = attention(q[None, a:b_], k[None, c:e], v[None, c:e], scale, causal)
        o[a:b_] = os_[0]
        lse[:, a:b_] = ls_[0]
    return o, lse


def decode(q, k, v, scale):
    """One query per sequence against a KV cache.

    q ``[B,Hq,d]``, cache ``[B,Skv,Hkv,d]`` -> o ``[B,Hq,d]``, lse ``[B,Hq]``.
    The query is the newest position, so every cached key is allowed.
    """
    o, lse = attention(q[:, None], k, v, scale, causal=False)
    return o[:, 0], lse[:, :, 0]


def decode_split(q, k, v, scale, num_splits):
    """Split-KV decode: attention over key chunks, then a log-sum-exp merge.

    The cache is cut into ``num_splits`` chunks of ``ceil(Skv/num_splits)``
    keys.  Each chunk gives a normalised partial output ``O_s`` and its
    ``lse_s``; the merge takes ``LSE = M + log(sum_s exp(lse_s - M))`` with
    ``M = max_s lse_s`` and ``O = sum_s exp(lse_s - LSE) * O_s``.  An empty
    chunk has ``lse_s = -inf`` and weight 0.  This is the same common-scale
    bookkeeping as the tiled softmax, applied once across chunks.
    """
    B, Skv = k.shape[0], k.shape[1]
    chunk = -(-Skv // num_splits)
    parts_o, parts_l = [], []
    for sp in range(num_splits):
        c0, c1 = sp * chunk, min(Skv, (sp + 1) * chunk)
        if c1 <= c0:
            parts_o.append(np.zeros(q.shape))
            parts_l.append(np.full(q.shape[:2], NEG_INF))
            continue
        os_, ls_ = decode(q, k[:, c0:c1], v[:, c0:c1], scale)
        parts_o.append(os_)
        parts_l.append(ls_)
    L = np.stack(parts_l)                      # [splits,B,Hq]
    M = L.max(axis=0)
    M_safe = np.where(np.isfinite(M), M, 0.0)
    w = np.exp(L - M_safe[None])
    tot = w.sum(axis=0)
    with np.errstate(divide="ignore"):
        lse = np.where(tot > 0, M_safe + np.log(np.where(tot > 0, tot, 1.0)), NEG_INF)
    o = (w[..., None] * np.stack(parts_o)).sum(axis=0) / np.where(tot > 0, tot, 1.0)[..., None]
    return o, lse


def e4m3fn_to_f64(codes):
    """FP8 E4M3 codes (uint8) -> float64, from the format's definition.

    The pages name FP8 among the formats each generation of matrix units
    adds (lecompute.fr, "Flapping Airplanes, ThunderKittens and megakernels",
    section "ThunderKittens starts with tiles, not whole applications",
    glossary note on Tensor Cores) but do not define it; this is the E4M3
    variant of the OCP 8-bit floating point specification (the "e4m3fn"
    layout): bit 7 is the sign, bits 6..3 the exponent field ``E`` with bias
    7, bits 2..0 the mantissa ``M``.

    * ``E == 0``: subnormal, ``(-1)^s * (M / 8) * 2^-6`` (so ``M == 0`` is a
      signed zero);
    * ``E == 15`` and ``M == 7``: NaN (the format has no infinities);
    * otherwise: normal, ``(-1)^s * (1 + M / 8) * 2^(E - 7)``; the largest
      magnitude is ``1.75 * 2^8 = 448``.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    val = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2((e - 7).astype(np.float64)))
    val = np.where((e == 15) & (c & 0x7 == 7), np.nan, val)
    return sign * val


def decode_fp8(q, k_codes, v_codes, scale, k_scale, v_scale, seqlens=None):
    """Decode against an FP8 (e4m3fn) KV cache.

    The cache stores codes and one scale per tensor: key ``j`` is
    ``k_scale * e4m3fn(k_codes[..., j, ...])`` and likewise for the values.
    The result is :func:`decode` over those dequantised values, sequence
    ``b`` seeing its first ``seqlens[b]`` keys (clamped to ``[0, Skv]``; all
    of them when ``seqlens`` is None).  A sequence with no key gets
    ``O = 0`` and ``LSE = -inf``.
    """
    k = e4m3fn_to_f64(k_codes) * float(k_scale)
    v = e4m3fn_to_f64(v_codes) * float(v_scale)
    q = np.asarray(q, dtype=np.float64)
    if seqlens is None:
        return decode(q, k, v, scale)
    B, Hq, d = q.shape
    Skv = k.shape[1]
    o = np.zeros((B, Hq, d))
    lse = np.full((B, Hq), NEG_INF)
    for b in range(B):
        n = min(max(int(seqlens[b]), 0), Skv)
        if n > 0:
            ob, lb = decode(q[b:b + 1], k[b:b + 1, :n], v[b:b + 1, :n], scale)
            o[b], lse[b] = ob[0], lb[0]
    return o, lse


def kmeans_distances(x, c):
    """Squared Euclidean distances ``D[n, k] = sum_i (x[n, i] - c[k, i])^2``.

    The assignment step of Lloyd's k-means compares every point with every
    centroid (lefilia.fr, "Flash-KMeans : un K-Means exact et optimisé pour
    les E/S, plus de 200 fois plus rapide que FAISS sur GPU", the paragraph
    on the assignment phase: each point goes to its nearest centroid).
    Written out from the definition, in float64, one point at a time, so no
    N x K x d temporary is formed.
    """
    x = np.asarray(x, dtype=np.float64)
    c = np.asarray(c, dtype=np.float64)
    out = np.empty((x.shape[0], c.shape[0]))
    for n in range(x.shape[0]):
        diff = c - x[n]
        out[n] = (diff * diff).sum(axis=1)
    return out


def kmeans_assign(x, c):
    """Nearest centroid of every point: ``idx[n] = argmin_k D[n, k]`` and
    ``dist[n] = D[n, idx[n]]``.

    Exact ties go to the lowest centroid index (the article stresses that
    the fused assignment gives exactly the result of the plain k-means;
    the lowest-index rule makes "the" nearest centroid unique).
    """
    D = kmeans_distances(x, c)
    idx = np.argmin(D, axis=1)          # first occurrence: lowest index on ties
    return idx, D[np.arange(D.shape[0]), idx]


def attention_rows(q, k, v, scale, causal, rows):
    """Selected output rows of :func:`attention`.

    ``rows`` is an int array ``[n,3]`` of ``(b, h, i)``; returns o ``[n,d]``
    and lse ``[n]``.  Each row is computed on its own from its score row, so
    very large workloads can be spot-checked.  Inputs may be bf16 bit arrays
    (uint16), widened one head slice at a time.
    """
    from_bits = q.dtype == np.uint16

    def wid(a):
        if from_bits:
            return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
        return np.asarray(a, dtype=np.float64)

    B, Sq, Hq, d = q.shape
    Skv, Hkv = k.shape[1], k.shape[2]
    g = Hq // Hkv
    rows = np.asarray(rows, dtype=np.int64).reshape(-1, 3)
    o = np.zeros((len(rows), d))
    lse = np.zeros(len(rows))
    for n, (b, h, i) in enumerate(rows):
        hk = h // g
        n_ok = Skv if not causal else min(Skv, max(0, i + (Skv - Sq) + 1))
        if n_ok == 0:
            lse[n] = NEG_INF
            continue
        kk = wid(k[b, :n_ok, hk, :])
        s = scale * (kk @ wid(q[b, i, h, :]))
        m = s.max()
        e = np.exp(s - m)
        l = e.sum()
        o[n] = (e @ wid(v[b, :n_ok, hk, :])) / l
        lse[n] = m + np.log(l)
    return o, lse
