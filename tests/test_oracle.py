"""Pins of the CPU oracle against what the pages and the mathematics fix.

The pages (lecompute.fr, "FlashAttention-4 : limites du calcul matriciel")
print no worked numeric example of attention, so the oracle is pinned by
closed forms, invariants, special cases that reduce to textbook routines,
a 50-digit brute force and equivalences the tiling argument promises.  Each
test names the mistake it is there to catch.
"""
import math

import numpy as np
import pytest

from oracle import cpu, ref
import synth_inputs as si


def rnd(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def bf16_arr(shape, seed):
    bits = si.f32_to_bf16_bits(np.random.default_rng(seed).standard_normal(shape).astype(np.float32))
    return bits, si.bf16_to_f64(bits)


CASES = [  # B, Sq, Skv, Hq, Hkv, d, causal
    (1, 5, 5, 1, 1, 4, False),
    (2, 7, 7, 4, 2, 8, True),
    (1, 3, 9, 2, 1, 8, True),     # Sq < Skv: bottom-right causal
    (2, 9, 4, 2, 2, 4, True),     # Sq > Skv: first rows fully masked
    (1, 6, 11, 3, 3, 5, False),
]


# ---- softmax weights: positive, sum to one (FA4 page, first section) ----

@pytest.mark.parametrize("case", CASES)
def test_weights_positive_and_sum_to_one(case):
    B, Sq, Skv, Hq, Hkv, d, causal = case
    q, k = rnd((B, Sq, Hq, d), 1), rnd((B, Skv, Hkv, d), 2)
    p = ref.attention_probs(q, k, 0.7, causal)
    ok = ref.allowed_mask(Sq, Skv, causal)
    assert np.all(p >= 0)
    assert np.all(p[..., ~ok] == 0)                       # nothing leaks past the mask
    rows_ok = ok.any(axis=1)
    s = p.sum(axis=-1)
    np.testing.assert_allclose(s[..., rows_ok], 1.0, atol=1e-14)
    assert np.all(s[..., ~rows_ok] == 0)
    assert np.all(p[..., ok] > 0)                        # every allowed key gets weight


# ---- closed forms ----

ALL_IMPLS = ["naive", "tiled", "c"]


def run_impl(impl, q, k, v, scale, causal):
    if impl == "naive":
        return ref.attention(q, k, v, scale, causal)
    if impl == "tiled":
        return ref.attention_tiled(q, k, v, scale, causal, br=3, bc=4)
    qb, kb, vb = (si.f32_to_bf16_bits(a.astype(np.float32)) for a in (q, k, v))
    assert np.array_equal(si.bf16_to_f64(qb), q) and np.array_equal(si.bf16_to_f64(vb), v)
    return cpu.attn_full(qb, kb, vb, scale, causal)


def bf16_exact(a):
    return si.bf16_to_f64(si.f32_to_bf16_bits(a.astype(np.float32)))


@pytest.mark.parametrize("impl", ALL_IMPLS)
@pytest.mark.parametrize("case", CASES)
def test_constant_v_gives_that_constant(impl, case):
    """V rows all equal c => every output row equals c (weights sum to one)."""
    B, Sq, Skv, Hq, Hkv, d, causal = case
    q, k = bf16_exact(rnd((B, Sq, Hq, d), 3)), bf16_exact(rnd((B, Skv, Hkv, d), 4))
    c = bf16_exact(rnd((d,), 5))
    v = np.broadcast_to(c, (B, Skv, Hkv, d)).copy()
    o, lse = run_impl(impl, q, k, v, 0.5, causal)
    rows_ok = ref.allowed_mask(Sq, Skv, causal).any(axis=1)
    np.testing.assert_allclose(o[:, rows_ok], np.broadcast_to(c, o[:, rows_ok].shape), atol=1e-13)
    assert np.all(o[:, ~rows_ok] == 0) and np.all(np.isneginf(lse[:, :, ~rows_ok]))


@pytest.mark.parametrize("impl", ALL_IMPLS)
@pytest.mark.parametrize("case", CASES)
def test_zero_query_gives_mean_and_log_count(impl, case):
    """q = 0 => uniform weights: O_i = mean of the allowed v_j, LSE_i = ln(#allowed).

    Catches an off-by-one in the causal limit and a wrong LSE base or offset.
    """
    B, Sq, Skv, Hq, Hkv, d, causal = case
    q = np.zeros((B, Sq, Hq, d))
    k, v = bf16_exact(rnd((B, Skv, Hkv, d), 6)), bf16_exact(rnd((B, Skv, Hkv, d), 7))
    o, lse = run_impl(impl, q, k, v, 0.3, causal)
    g = Hq // Hkv
    for i in range(Sq):
        n = Skv if not causal else max(0, min(Skv, i + Skv - Sq + 1))
        for h in range(Hq):
            if n == 0:
                assert np.all(o[:, i, h] == 0) and np.all(np.isneginf(lse[:, h, i]))
                continue
            np.testing.assert_allclose(o[:, i, h], v[:, :n, h // g].mean(axis=1), atol=1e-13)
            np.testing.assert_allclose(lse[:, h, i], math.log(n), atol=1e-13)


@pytest.mark.parametrize("impl", ALL_IMPLS)
def test_huge_score_selects_one_value_row(impl):
    """One key with a score far above the rest: O_i = v_j and LSE_i ~= that score.

    Exercises the max subtraction (the page's point that an overflowed value
    cannot be repaired afterwards): exp(1000) would overflow without it.
    """
    B, S, H, d = 1, 6, 1, 8
    k = np.zeros((B, S, H, d))
    k[0, :, 0, :S] = np.eye(S)                     # near-orthogonal keys
    k = bf16_exact(k + 0.01 * rnd((B, S, H, d), 8))
    v = bf16_exact(rnd((B, S, H, d), 9))
    q = np.zeros((B, S, H, d))
    target = [2, 0, 5, 3, 1, 4]
    for i, j in enumerate(target):
        q[0, i, 0] = 1000.0 * k[0, j, 0] / np.dot(k[0, j, 0], k[0, j, 0])
    q = bf16_exact(q)
    o, lse = run_impl(impl, q, k, v, 1.0, False)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    for i, j in enumerate(target):
        np.testing.assert_allclose(o[0, i, 0], v[0, j, 0], atol=1e-12)
        s = q[0, i, 0] @ k[0, :, 0].T
        assert s[j] > 900 and s[j] - np.delete(s, j).max() > 100
        np.testing.assert_allclose(lse[0, 0, i], s[j], atol=1e-12)


@pytest.mark.parametrize("impl", ALL_IMPLS)
def test_causal_first_row_sees_only_first_key(impl):
    """Causal, Sq = Skv: row 0 => O_0 = v_0 and LSE_0 = scale * q_0.k_0 exactly."""
    q, k, v = (bf16_exact(rnd((2, 5, 2, 8), s)) for s in (10, 11, 12))
    o, lse = run_impl(impl, q, k, v, 0.25, True)
    np.testing.assert_allclose(o[:, 0], v[:, 0], atol=1e-15)
    np.testing.assert_allclose(lse[:, :, 0], 0.25 * np.einsum("bhd,bhd->bh", q[:, 0], k[:, 0]),
                               atol=1e-13)


@pytest.mark.parametrize("impl", ALL_IMPLS)
def test_two_keys_reduce_to_logistic(impl):
    """Skv = 2: the weight of key 0 is the logistic function of s_0 - s_1."""
    from scipy.special import expit
    q, k, v = (bf16_exact(rnd(sh, s)) for sh, s in (((1, 4, 1, 8), 13), ((1, 2, 1, 8), 14),
                                                       ((1, 2, 1, 8), 15)))
    o, lse = run_impl(impl, q, k, v, 0.4, False)
    s = 0.4 * q[0, :, 0] @ k[0, :, 0].T
    w0 = expit(s[:, 0] - s[:, 1])
    np.testing.assert_allclose(o[0, :, 0], w0[:, None] * v[0, 0, 0] + (1 - w0)[:, None] * v[0, 1, 0],
                               atol=1e-13)
    np.testing.assert_allclose(lse[0, 0], np.logaddexp(s[:, 0], s[:, 1]), atol=1e-13)


def test_hand_worked_three_to_one():
    """Scores (ln 3, 0) give weights (3/4, 1/4) and LSE = ln 4 (worked by hand)."""
    q = np.array([[[[1.0, 0.0]]]])
    k = np.array([[[[math.log(3.0), 0.0]], [[0.0, 5.0]]]])
    v = np.array([[[[8.0, -4.0]], [[4.0, 12.0]]]])
    for o, lse in (ref.attention(q, k, v, 1.0), ref.attention_tiled(q, k, v, 1.0, br=1, bc=1)):
        np.testing.assert_allclose(o[0, 0, 0], [7.0, 0.0], atol=1e-14)
        np.testing.assert_allclose(lse[0, 0, 0], math.log(4.0), atol=1e-14)


# ---- invariants ----

@pytest.mark.parametrize("impl", ALL_IMPLS)
def test_noncausal_key_permutation_invariance(impl):
    """Non-causal: permuting K and V rows together changes nothing."""
    q, k, v = (bf16_exact(rnd(sh, s)) for sh, s in (((2, 6, 4, 8), 16), ((2, 9, 2, 8), 17),
                                                       ((2, 9, 2, 8), 18)))
    perm = np.random.default_rng(19).permutation(9)
    o1, l1 = run_impl(impl, q, k, v, 0.35, False)
    o2, l2 = run_impl(impl, q, k[:, perm], v[:, perm], 0.35, False)
    np.testing.assert_allclose(o1, o2, atol=1e-13)
    np.testing.assert_allclose(l1, l2, atol=1e-13)
    o3, _ = run_impl(impl, q, k[:, perm], v[:, perm], 0.35, True)
    o4, _ = run_impl(impl, q, k, v, 0.35, True)
    assert np.abs(o3 - o4).max() > 1e-3     # the causal path must notice the order


def test_score_shift_moves_lse_only():
    """Adding the same amount to every score of a row leaves O and shifts LSE by it.

    Built with a key feature that is 1 for every key: raising q's matching
    entry by t adds scale*t to all scores of that row.
    """
    B, Sq, Skv, H, d = 1, 5, 7, 2, 6
    q, k, v = rnd((B, Sq, H, d), 20), rnd((B, Skv, H, d), 21), rnd((B, Skv, H, d), 22)
    k[..., 0] = 1.0
    for causal in (False, True):
        o1, l1 = ref.attention(q, k, v, 0.5, causal)
        q2 = q.copy()
        q2[..., 0] += 3.0
        o2, l2 = ref.attention(q2, k, v, 0.5, causal)
        np.testing.assert_allclose(o1, o2, atol=1e-13)
        np.testing.assert_allclose(l2 - l1, 1.5, atol=1e-13)


def test_scale_acts_on_scores_only():
    """scale * (q.k) == (scale q).k: the scale multiplies scores, not values."""
    q, k, v = rnd((1, 6, 2, 8), 23), rnd((1, 6, 2, 8), 24), rnd((1, 6, 2, 8), 25)
    o1, l1 = ref.attention(q, k, v, 0.37, True)
    o2, l2 = ref.attention(q * 0.37, k, v, 1.0, True)
    np.testing.assert_allclose(o1, o2, atol=1e-13)
    np.testing.assert_allclose(l1, l2, atol=1e-13)


def test_gqa_equals_mha_with_repeated_kv():
    """GQA with group g equals MHA whose KV heads are repeated g times (consecutive)."""
    q, k, v = rnd((2, 5, 6, 4), 26), rnd((2, 8, 2, 4), 27), rnd((2, 8, 2, 4), 28)
    for causal in (False, True):
        o1, l1 = ref.attention(q, k, v, 0.5, causal)
        o2, l2 = ref.attention(q, np.repeat(k, 3, axis=2), np.repeat(v, 3, axis=2), 0.5, causal)
        np.testing.assert_allclose(o1, o2, atol=1e-15)
        np.testing.assert_allclose(l1, l2, atol=1e-15)
    # and not the interleaved grouping
    o3, _ = ref.attention(q, np.tile(k, (1, 1, 3, 1)), np.tile(v, (1, 1, 3, 1)), 0.5, False)
    o1, _ = ref.attention(q, k, v, 0.5, False)
    assert np.abs(o1 - o3).max() > 1e-3


# ---- tiling equivalence (FA4 page: tiles give the same result) ----

@pytest.mark.parametrize("br,bc", [(1, 1), (3, 5), (7, 2), (16, 16), (5, 100), (2, 3)])
@pytest.mark.parametrize("case", CASES)
def test_tiled_online_softmax_equals_naive(br, bc, case):
    B, Sq, Skv, Hq, Hkv, d, causal = case
    q, k, v = rnd((B, Sq, Hq, d), 30, 3.0), rnd((B, Skv, Hkv, d), 31), rnd((B, Skv, Hkv, d), 32)
    o1, l1 = ref.attention(q, k, v, 0.9, causal)
    o2, l2 = ref.attention_tiled(q, k, v, 0.9, causal, br=br, bc=bc)
    np.testing.assert_allclose(o1, o2, atol=1e-12, rtol=0)
    fin = np.isfinite(l1)
    assert np.array_equal(fin, np.isfinite(l2))
    np.testing.assert_allclose(l1[fin], l2[fin], atol=1e-12, rtol=0)


def test_tiled_handles_growing_max_without_overflow():
    """Scores that rise by hundreds from tile to tile still give finite results."""
    S, d = 12, 4
    k = np.zeros((1, S, 1, d))
    k[0, :, 0, 0] = np.arange(S) * 60.0         # later keys score much higher
    q = np.zeros((1, S, 1, d))
    q[0, :, 0, 0] = 1.0
    v = rnd((1, S, 1, d), 33)
    o1, l1 = ref.attention(q, k, v, 1.0, True)
    o2, l2 = ref.attention_tiled(q, k, v, 1.0, True, br=4, bc=2)
    assert np.all(np.isfinite(o2)) and np.all(np.isfinite(l2))
    np.testing.assert_allclose(o1, o2, atol=1e-12)
    np.testing.assert_allclose(l1, l2, atol=1e-10)
    np.testing.assert_allclose(o2[0, :, 0], v[0, :, 0], atol=1e-12)  # the diagonal key wins


# ---- exact arithmetic on tiny inputs ----

def _mp_attention(q, k, v, scale, causal, dps=50):
    import mpmath as mp
    mp.mp.dps = dps
    Sq, Skv, d = q.shape[0], k.shape[0], q.shape[1]
    o = [[None] * d for _ in range(Sq)]
    lse = [None] * Sq
    sc = mp.mpf(scale)
    for i in range(Sq):
        lim = Skv if not causal else i + (Skv - Sq) + 1
        s = [sc * mp.fsum(mp.mpf(float(q[i, c])) * mp.mpf(float(k[j, c])) for c in range(d))
             for j in range(lim)]
        z = mp.fsum(mp.e ** x for x in s)
        for c in range(d):
            o[i][c] = mp.fsum(mp.e ** s[j] * mp.mpf(float(v[j, c])) for j in range(lim)) / z
        lse[i] = mp.log(z)
    return o, lse


@pytest.mark.parametrize("causal", [False, True])
def test_fifty_digit_brute_force(causal):
    """fp64 oracle (numpy and C) vs 50-digit mpmath on tiny inputs: <= 1e-13."""
    qb, q = bf16_arr((1, 4, 2, 5), 34)
    kb, k = bf16_arr((1, 6, 1, 5), 35)
    vb, v = bf16_arr((1, 6, 1, 5), 36)
    on, ln = ref.attention(q, k, v, 0.6, causal)
    oc, lc = cpu.attn_full(qb, kb, vb, 0.6, causal)
    for h in range(2):
        o_mp, l_mp = _mp_attention(q[0, :, h], k[0, :, 0], v[0, :, 0], 0.6, causal)
        for i in range(4):
            for c in range(5):
                assert abs(on[0, i, h, c] - float(o_mp[i][c])) < 1e-13
                assert abs(oc[0, i, h, c] - float(o_mp[i][c])) < 1e-13
            assert abs(ln[0, h, i] - float(l_mp[i])) < 1e-13
            assert abs(lc[0, h, i] - float(l_mp[i])) < 1e-13


def test_plain_python_loops():
    """A pure-Python loop transcription (math.exp) agrees with numpy to 1e-13."""
    q, k, v = rnd((3, 4), 37), rnd((5, 4), 38), rnd((5, 4), 39)
    o, lse = ref.attention(q[None, :, None], k[None, :, None], v[None, :, None], 0.8, True)
    for i in range(3):
        lim = i + 2 + 1
        s = [0.8 * sum(q[i, c] * k[j, c] for c in range(4)) for j in range(lim)]
        z = sum(math.exp(x) for x in s)
        for c in range(4):
            assert abs(sum(math.exp(s[j]) * v[j, c] for j in range(lim)) / z - o[0, i, 0, c]) < 1e-13
        assert abs(math.log(z) - lse[0, 0, i]) < 1e-13


# ---- masks at the edges ----

def test_fully_masked_rows_when_more_queries_than_keys():
    """Sq > Skv, causal, bottom-right: rows i < Sq-Skv see nothing -> O=0, LSE=-inf."""
    q, k, v = rnd((1, 6, 1, 4), 40), rnd((1, 2, 1, 4), 41), rnd((1, 2, 1, 4), 42)
    o, lse = ref.attention(q, k, v, 1.0, True)
    assert np.all(o[0, :4] == 0) and np.all(np.isneginf(lse[0, 0, :4]))
    np.testing.assert_allclose(o[0, 4, 0], v[0, 0, 0], atol=1e-15)   # sees key 0 only
    assert np.all(np.isfinite(lse[0, 0, 4:]))


def test_decode_is_last_row_and_sees_whole_cache():
    """Bottom-right alignment: one query attends to every cached key."""
    q, k, v = rnd((3, 4, 8), 43), rnd((3, 10, 2, 8), 44), rnd((3, 10, 2, 8), 45)
    o, lse = ref.decode(q, k, v, 0.5)
    o2, l2 = ref.attention(q[:, None], k, v, 0.5, causal=True)
    np.testing.assert_allclose(o, o2[:, 0], atol=1e-15)
    np.testing.assert_allclose(lse, l2[:, :, 0], atol=1e-15)
    # the same query as the last row of a full causal prefill
    qf = rnd((3, 10, 4, 8), 46)
    qf[:, -1] = q
    of, lf = ref.attention(qf, k, v, 0.5, causal=True)
    np.testing.assert_allclose(o, of[:, -1], atol=1e-13)


@pytest.mark.parametrize("splits", [1, 2, 3, 8, 10, 16])
def test_split_kv_merge_equals_decode(splits):
    """Chunked partials merged by log-sum-exp equal one pass (empty chunks included)."""
    q, k, v = rnd((2, 4, 8), 47, 2.0), rnd((2, 10, 2, 8), 48), rnd((2, 10, 2, 8), 49)
    o1, l1 = ref.decode(q, k, v, 0.7)
    o2, l2 = ref.decode_split(q, k, v, 0.7, splits)
    np.testing.assert_allclose(o1, o2, atol=1e-13)
    np.testing.assert_allclose(l1, l2, atol=1e-13)


def test_varlen_equals_separate_calls_and_c_rows():
    lengths = [3, 1, 8, 5]
    data = si.make_varlen(50, 4, 1, 8, H=4, d=8, Hkv=2, lengths=lengths)
    q, k, v = (si.bf16_to_f64(data[x]) for x in "qkv")
    cu = data["cu_seqlens"]
    for causal in (False, True):
        o, lse = ref.attention_varlen(q, k, v, cu, cu, 0.5, causal)
        for s in range(4):
            a, b = cu[s], cu[s + 1]
            os_, ls_ = ref.attention(q[None, a:b], k[None, a:b], v[None, a:b], 0.5, causal)
            np.testing.assert_array_equal(o[a:b], os_[0])
            np.testing.assert_array_equal(lse[:, a:b], ls_[0])
        rows = np.array([(s, h, i) for s in range(4) for h in range(4) for i in range(lengths[s])])
        oc, lc = cpu.varlen_rows(data["q"], data["k"], data["v"], cu, cu, 0.5, causal, rows)
        for n, (s, h, i) in enumerate(rows):
            np.testing.assert_allclose(oc[n], o[cu[s] + i, h], atol=1e-13)
            np.testing.assert_allclose(lc[n], lse[h, cu[s] + i], atol=1e-13)


def test_varlen_cross_lengths_and_empty_sequences():
    """Chunked-prefill shape: query and key lengths differ per sequence.

    A sequence with no keys gives O = 0 and LSE = -inf on every row (the
    no-allowed-key reading); a sequence with no queries writes nothing.  Each
    non-empty sequence equals a separate call, under bottom-right causal
    alignment, and the C oracle's rows agree with the numpy ones.
    """
    lq, lk = [2, 0, 5, 3, 1], [4, 3, 5, 0, 6]
    data = si.make_varlen_cross(57, lq, lk, H=4, d=8, Hkv=2)
    q, k, v = (si.bf16_to_f64(data[x]) for x in "qkv")
    cq, ck = data["cu_seqlens_q"], data["cu_seqlens_k"]
    for causal in (False, True):
        o, lse = ref.attention_varlen(q, k, v, cq, ck, 0.5, causal)
        # sequence 3 has three queries and no keys
        assert np.all(o[cq[3]:cq[4]] == 0) and np.all(np.isneginf(lse[:, cq[3]:cq[4]]))
        for s in (0, 2, 4):
            a, b, c, e = cq[s], cq[s + 1], ck[s], ck[s + 1]
            os_, ls_ = ref.attention(q[None, a:b], k[None, c:e], v[None, c:e], 0.5, causal)
            np.testing.assert_array_equal(o[a:b], os_[0])
            np.testing.assert_array_equal(lse[:, a:b], ls_[0])
        if causal:
            # sequence 0: 2 queries after 2 earlier keys; row 0 sees keys 0..2
            s_ = 0.5 * (q[0, 0] @ k[0:3, 0].T)
            w = np.exp(s_ - s_.max())
            np.testing.assert_allclose(o[0, 0], (w / w.sum()) @ v[0:3, 0], atol=1e-14)
        rows = np.array([(s, h, i) for s in range(5) for h in range(4) for i in range(lq[s])])
        oc, lc = cpu.varlen_rows(data["q"], data["k"], data["v"], cq, ck, 0.5, causal, rows)
        for n, (s, h, i) in enumerate(rows):
            np.testing.assert_allclose(oc[n], o[cq[s] + i, h], atol=1e-13)
            assert lc[n] == lse[h, cq[s] + i] or abs(lc[n] - lse[h, cq[s] + i]) < 1e-13


# ---- the C oracle against the numpy oracle, and sampled rows ----

@pytest.mark.parametrize("case", CASES)
def test_c_oracle_matches_numpy(case):
    B, Sq, Skv, Hq, Hkv, d, causal = case
    qb, q = bf16_arr((B, Sq, Hq, d), 51)
    kb, k = bf16_arr((B, Skv, Hkv, d), 52)
    vb, v = bf16_arr((B, Skv, Hkv, d), 53)
    o1, l1 = ref.attention(q, k, v, 0.45, causal)
    o2, l2 = cpu.attn_full(qb, kb, vb, 0.45, causal)
    np.testing.assert_allclose(o1, o2, atol=1e-13)
    assert np.array_equal(np.isfinite(l1), np.isfinite(l2))
    f = np.isfinite(l1)
    np.testing.assert_allclose(l1[f], l2[f], atol=1e-13)
    rows = np.array([[B - 1, Hq - 1, Sq - 1], [0, 0, 0], [0, Hq // 2, Sq // 2]])
    o3, l3 = ref.attention_rows(qb, kb, vb, 0.45, causal, rows)
    for n, (b, h, i) in enumerate(rows):
        np.testing.assert_allclose(o3[n], o1[b, i, h], atol=1e-13)
        if np.isfinite(l1[b, h, i]):
            assert abs(l3[n] - l1[b, h, i]) < 1e-13


def test_c_oracle_rejects_bad_arguments():
    qb, _ = bf16_arr((1, 2, 3, 4), 54)
    kb, _ = bf16_arr((1, 2, 2, 4), 55)
    with pytest.raises(ValueError):            # Hq not a multiple of Hkv
        cpu.attn_rows(qb, kb, kb, 1.0, False, [[0, 0, 0]])
    qb, _ = bf16_arr((1, 2, 2, 4), 56)
    with pytest.raises(ValueError):            # row out of range
        cpu.attn_rows(qb, kb, kb, 1.0, False, [[0, 2, 0]])


# ----------------------------------------------------------- fp8 KV cache

def test_e4m3fn_closed_form_values():
    """Codes whose values the E4M3 definition fixes by hand."""
    cases = {
        0x00: 0.0, 0x80: -0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6,
        0x38: 1.0, 0x39: 1.125, 0x3F: 1.875, 0x40: 2.0, 0x30: 0.5, 0xB8: -1.0, 0xC0: -2.0,
        0x77: 240.0, 0x78: 256.0, 0x7E: 448.0, 0xFE: -448.0,
    }
    codes = np.array(sorted(cases), dtype=np.uint8)
    got = ref.e4m3fn_to_f64(codes)
    want = np.array([cases[c] for c in sorted(cases)])
    assert np.array_equal(got, want)
    assert np.signbit(ref.e4m3fn_to_f64(np.array([0x80], dtype=np.uint8)))[0]
    nan = ref.e4m3fn_to_f64(np.array([0x7F, 0xFF], dtype=np.uint8))
    assert np.all(np.isnan(nan))


def test_e4m3fn_matches_torch_on_every_code():
    """All 256 codes against torch's own float8_e4m3fn -> float64 widening."""
    import torch
    codes = np.arange(256, dtype=np.uint8)
    ours = ref.e4m3fn_to_f64(codes)
    theirs = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(theirs)
    assert np.array_equal(np.isnan(ours), nan) and nan.sum() == 2
    assert np.array_equal(ours[~nan], theirs[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(theirs[~nan]))


def test_e4m3fn_order_and_symmetry():
    """Codes 0..0x7E increase strictly; the sign bit only flips the sign."""
    pos = ref.e4m3fn_to_f64(np.arange(0x7F, dtype=np.uint8))
    assert np.all(np.diff(pos) > 0)
    neg = ref.e4m3fn_to_f64(np.arange(0x80, 0xFF, dtype=np.uint8))
    assert np.array_equal(neg, -pos)


def _fp8_case(seed=5, B=3, Hq=4, Hkv=2, Skv=37, d=16):
    data = si.make_decode_fp8(seed, B, Hq, Hkv, Skv, d)
    return data, si.bf16_to_f64(data["q"])


def test_decode_fp8_scales_enter_where_stated():
    """O is linear in v_scale with LSE unchanged; only scale * k_scale matters."""
    data, q = _fp8_case()
    o1, l1 = ref.decode_fp8(q, data["k"], data["v"], 0.25, 0.5, 0.75)
    o2, l2 = ref.decode_fp8(q, data["k"], data["v"], 0.25, 0.5, 1.5)
    assert np.allclose(o2, 2 * o1, rtol=1e-13, atol=0) and np.array_equal(l1, l2)
    o3, l3 = ref.decode_fp8(q, data["k"], data["v"], 0.5, 0.25, 0.75)
    assert np.allclose(o3, o1, rtol=1e-12, atol=1e-14) and np.allclose(l3, l1, rtol=1e-13)


def test_decode_fp8_uniform_keys_give_value_mean():
    """Every key code 1.0: all scores equal q.1 * scale * k_scale, so O is the mean
    dequantised value row and LSE = log(n) + that score (closed form)."""
    data, q = _fp8_case()
    k = np.full_like(data["k"], 0x38)
    scale, ks, vs = 0.3, 0.125, 0.0625
    o, lse = ref.decode_fp8(q, k, data["v"], scale, ks, vs)
    B, Hq, d = q.shape
    Skv, Hkv = k.shape[1], k.shape[2]
    g = Hq // Hkv
    vd = ref.e4m3fn_to_f64(data["v"]) * vs
    for b in range(B):
        for h in range(Hq):
            want_o = vd[b, :, h // g, :].mean(axis=0)
            want_l = math.log(Skv) + scale * ks * q[b, h].sum()
            assert np.allclose(o[b, h], want_o, rtol=1e-12, atol=1e-15)
            assert abs(lse[b, h] - want_l) < 1e-12


def test_decode_fp8_lengths_are_prefixes_and_clamped():
    """A length picks a prefix of the cache; 0 gives O = 0, LSE = -inf; out-of-range
    lengths clamp to [0, Skv]."""
    data, q = _fp8_case(B=4)
    lens = np.array([0, 5, 37, 99])
    o, lse = ref.decode_fp8(q, data["k"], data["v"], 0.2, 1.0, 1.0, seqlens=lens)
    assert np.all(o[0] == 0) and np.all(np.isneginf(lse[0]))
    o5, l5 = ref.decode_fp8(q[1:2], data["k"][1:2, :5], data["v"][1:2, :5], 0.2, 1.0, 1.0)
    assert np.array_equal(o[1], o5[0]) and np.array_equal(lse[1], l5[0])
    full, lf = ref.decode_fp8(q, data["k"], data["v"], 0.2, 1.0, 1.0)
    assert np.array_equal(o[2:], full[2:]) and np.array_equal(lse[2:], lf[2:])
    neg, ln = ref.decode_fp8(q, data["k"], data["v"], 0.2, 1.0, 1.0, seqlens=[-3, 0, 0, 0])
    assert np.all(neg == 0) and np.all(np.isneginf(ln))


def test_decode_fp8_brute_force_one_row():
    """One output row by plain Python loops from the code values."""
    data, q = _fp8_case(B=1, Hq=2, Hkv=1, Skv=6, d=4)
    scale, ks, vs = 0.7, 0.05, 0.02
    o, lse = ref.decode_fp8(q, data["k"], data["v"], scale, ks, vs)
    kd = ref.e4m3fn_to_f64(data["k"])
    vd = ref.e4m3fn_to_f64(data["v"])
    for h in range(2):
        s = [scale * sum(q[0, h, t] * ks * kd[0, j, 0, t] for t in range(4)) for j in range(6)]
        m = max(s)
        w = [math.exp(x - m) for x in s]
        tot = sum(w)
        for t in range(4):
            want = sum(w[j] * vs * vd[0, j, 0, t] for j in range(6)) / tot
            assert abs(o[0, h, t] - want) < 1e-12
        assert abs(lse[0, h] - (m + math.log(tot))) < 1e-12


# ------------------------------------------------- k-means assignment

def _km(seed=3, N=200, K=37, d=16):
    data = si.make_kmeans(seed, N, K, d)
    return si.bf16_to_f64(data["x"]), si.bf16_to_f64(data["c"])


def test_kmeans_brute_force_python_loops():
    """Nearest centroid by plain Python loops over points, centroids and coordinates."""
    x, c = _km(N=25, K=9, d=5)
    idx, dist = ref.kmeans_assign(x, c)
    for n in range(25):
        best, best_k = None, None
        for k in range(9):
            s = 0.0
            for i in range(5):
                s += (x[n, i] - c[k, i]) ** 2
            if best is None or s < best:
                best, best_k = s, k
        assert idx[n] == best_k and abs(dist[n] - best) <= 1e-12 * max(1.0, best)


def test_kmeans_distance_expansion_identity():
    """|x - c|^2 = |x|^2 + |c|^2 - 2 x.c (checked through a matrix product)."""
    x, c = _km()
    D = ref.kmeans_distances(x, c)
    E = (x * x).sum(1)[:, None] + (c * c).sum(1)[None, :] - 2.0 * (x @ c.T)
    assert np.allclose(D, E, rtol=1e-12, atol=1e-10)
    assert np.all(D >= 0)


def test_kmeans_one_dimension_nearest_on_a_line():
    """d = 1: the nearest centroid found by bisection in the sorted centroid list."""
    rng = np.random.default_rng(4)
    c = np.unique(rng.standard_normal(50))[:, None]          # sorted, distinct
    x = rng.standard_normal(400)[:, None] * 1.5
    idx, dist = ref.kmeans_assign(x, c)
    cs = c[:, 0]
    j = np.clip(np.searchsorted(cs, x[:, 0]), 1, len(cs) - 1)
    left, right = cs[j - 1], cs[j]
    pick = np.where(np.abs(x[:, 0] - left) <= np.abs(right - x[:, 0]), j - 1, j)
    assert np.array_equal(idx, pick)
    assert np.allclose(dist, (x[:, 0] - cs[pick]) ** 2, rtol=0, atol=1e-15)


def test_kmeans_ties_go_to_the_lowest_index():
    """Duplicated centroids: the first copy wins; a point on a centroid has distance 0."""
    x, c = _km(N=60, K=10, d=8)
    c2 = np.concatenate([c[:3], c[5:6], c[3:]])              # centroid 5 also at index 3
    idx, dist = ref.kmeans_assign(x, c2)
    base, bd = ref.kmeans_assign(x, c)
    want = np.where(base < 3, base, np.where(base == 5, 3, base + 1))
    assert np.array_equal(idx, want) and np.array_equal(dist, bd)
    on, d0 = ref.kmeans_assign(c2[[6, 3, 0]], c2)
    assert list(on) == [3, 3, 0] and np.all(d0 == 0)


def test_kmeans_permutation_translation_and_scaling():
    """Relabelled centroids relabel the answer; a common shift or scale changes
    no assignment (scale a multiplies the distances by a^2)."""
    x, c = _km()
    idx, dist = ref.kmeans_assign(x, c)
    perm = np.random.default_rng(5).permutation(c.shape[0])
    ip, dp = ref.kmeans_assign(x, c[perm])
    assert np.array_equal(perm[ip], idx) and np.allclose(dp, dist, rtol=1e-13)
    t = np.random.default_rng(6).standard_normal(c.shape[1]) * 3
    it, dt = ref.kmeans_assign(x + t, c + t)
    assert np.array_equal(it, idx) and np.allclose(dt, dist, rtol=1e-9, atol=1e-9)
    isc, dsc = ref.kmeans_assign(4.0 * x, 4.0 * c)
    assert np.array_equal(isc, idx) and np.allclose(dsc, 16.0 * dist, rtol=1e-13)


def test_kmeans_mixture_recovers_labels():
    """Well separated mixture (the input recipe): every point goes to its own component."""
    data = si.make_kmeans(8, 500, 20, 64)
    idx, _ = ref.kmeans_assign(si.bf16_to_f64(data["x"]), si.bf16_to_f64(data["c"]))
    assert np.array_equal(idx, data["label"])
