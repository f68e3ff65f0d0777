"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

O (bf16) must be within 2e-2 max-abs of the unrounded fp64 oracle and LSE
(fp32) within 1e-3, on the same seeded bf16 inputs.  Small cases compare
every output; the five workloads at full size compare sampled rows that the
oracle computes one by one, in the same launch configuration the benchmark
times.
"""
import numpy as np
import pytest

import synth_inputs as si
from oracle import cpu, ref
from tests.gpu_util import (assert_close, bf16_to_np, decode_varlen_ref, f32_to_np, sample_rows,
                            to_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def api():
    from tiled_attention_transformer_amd import api as a
    a._lib.load()
    return a


def run_fwd(api, dev, data, scale, causal):
    import torch
    q, k, v = (to_dev(data[n], dev) for n in "qkv")
    o, lse = api.attn_fwd(q, k, v, scale=scale, causal=causal)
    torch.cuda.synchronize()
    return bf16_to_np(o), f32_to_np(lse)


# ---------------------------------------------------------------- small, whole

SMALL = [  # B, Sq, Skv, Hq, Hkv, d, causal
    (1, 256, 256, 2, 2, 64, False),
    (1, 300, 300, 2, 1, 128, True),      # ragged last query tile and key tile
    (2, 129, 257, 4, 2, 64, True),       # Sq < Skv, bottom-right causal
    (1, 200, 77, 2, 2, 128, True),       # Sq > Skv: leading rows fully masked
    (1, 200, 77, 2, 2, 64, False),
    (1, 1, 300, 4, 1, 128, False),       # a single query row
    (1, 1, 1, 1, 1, 64, True),           # smallest case
    (2, 384, 384, 8, 8, 128, True),      # several full tiles
    (1, 33, 500, 8, 2, 128, False),
    (1, 130, 130, 4, 4, 64, True),
    (3, 65, 200, 6, 3, 128, False),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "B%d_Sq%d_Skv%d_Hq%d_Hkv%d_d%d_%s" % (
    *c[:6], "causal" if c[6] else "full"))
def test_small_prefill_matches_oracle(api, dev, case):
    B, Sq, Skv, Hq, Hkv, d, causal = case
    data = si.make_prefill(100 + Sq + Skv, B, Hq, Hkv, Sq, Skv, d)
    scale = si.default_scale(d)
    o, lse = run_fwd(api, dev, data, scale, causal)
    o_ref, lse_ref = cpu.attn_full(data["q"], data["k"], data["v"], scale, causal)
    assert_close(o, o_ref, lse, lse_ref, str(case))
    if causal and Sq > Skv:
        assert np.all(o[:, :Sq - Skv] == 0)


# Batches wide enough for 256-row items on 8-wave workgroups (at least one
# item per CU of a 256-CU GPU); the cases above, with fewer items, run
# 128-row items on 4-wave workgroups.  Both paths compute each row the same
# way; these pin the wide path's edges.
WIDE = [  # B, Sq, Skv, Hq, Hkv, d, causal
    (16, 300, 300, 16, 16, 128, True),    # ragged last query and key tiles
    (16, 200, 77, 16, 8, 64, True),       # Sq > Skv: leading rows fully masked
    (16, 129, 257, 16, 4, 128, True),     # Sq < Skv, bottom-right causal
    (8, 260, 333, 32, 8, 128, False),
]


@pytest.mark.parametrize("case", WIDE, ids=lambda c: "B%d_Sq%d_Skv%d_Hq%d_Hkv%d_d%d_%s" % (
    *c[:6], "causal" if c[6] else "full"))
def test_wide_batch_prefill_matches_oracle(api, dev, case):
    B, Sq, Skv, Hq, Hkv, d, causal = case
    data = si.make_prefill(300 + Sq + Skv, B, Hq, Hkv, Sq, Skv, d)
    scale = si.default_scale(d)
    o, lse = run_fwd(api, dev, data, scale, causal)
    o_ref, lse_ref = cpu.attn_full(data["q"], data["k"], data["v"], scale, causal)
    assert_close(o, o_ref, lse, lse_ref, str(case))
    if causal and Sq > Skv:
        assert np.all(o[:, :Sq - Skv] == 0)


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_wide_and_small_grid_paths_agree_bitwise(api, dev, causal):
    """A 16-sequence batch runs 256-row items on 8-wave workgroups; its first
    sequence alone (fewer items than CUs) runs 128-row items on 4-wave ones.
    Each row is computed the same way, so the shared rows match bit for bit;
    the same holds for a ragged batch and its first sequence."""
    import torch
    B, S, Hq, Hkv, d = 16, 700, 16, 4, 128
    data = si.make_prefill(81, B, Hq, Hkv, S, S, d)
    q, k, v = (to_dev(data[x], dev) for x in "qkv")
    o_all, l_all = api.attn_fwd(q, k, v, causal=causal)
    o_one, l_one = api.attn_fwd(q[:1].contiguous(), k[:1].contiguous(), v[:1].contiguous(),
                                causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o_all[:1].view(torch.int16), o_one.view(torch.int16))
    assert torch.equal(l_all[:1], l_one)
    # ragged: 16 sequences of 700 tokens packed, against the first one alone
    qv, kv, vv = (t.reshape(B * S, t.shape[2], d) for t in (q, k, v))
    cu = torch.arange(0, (B + 1) * S, S, dtype=torch.int32, device=dev)
    o_r, l_r = api.attn_fwd_varlen(qv, kv, vv, cu, cu, S, S, causal=causal)
    cu1 = cu[:2].contiguous()
    o_r1, l_r1 = api.attn_fwd_varlen(qv[:S].contiguous(), kv[:S].contiguous(), vv[:S].contiguous(),
                                     cu1, cu1, S, S, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o_r[:S].view(torch.int16), o_r1.view(torch.int16))
    assert torch.equal(l_r[:, :S], l_r1)
    assert torch.equal(o_r[:S].view(torch.int16), o_one[0].view(torch.int16))


def _golden(name):
    import json
    import os
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", name)
    return json.load(open(path))


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_tiny_config_whole_and_golden(api, dev, causal):
    """Workload 1 (B1 H2 S256 d64) compared in full with the numpy oracle,
    and the stored oracle rows of tests/golden/ compared with the kernel's."""
    spec, data = si.make_workload("tiny")
    o, lse = run_fwd(api, dev, data, spec["scale"], causal)
    o_ref, lse_ref = ref.attention(*(si.bf16_to_f64(data[n]) for n in "qkv"), spec["scale"],
                                   causal)
    assert_close(o, o_ref, lse, lse_ref, "workload 1")
    g = _golden("tiny_%s_rows.json" % ("causal" if causal else "noncausal"))
    assert g["causal"] == causal and g["scale"] == spec["scale"]
    rows = np.array(g["rows"], dtype=np.int64)
    b, h, i = rows[:, 0], rows[:, 1], rows[:, 2]
    assert_close(o[b, i, h], np.array(g["o"]), lse[b, h, i], np.array(g["lse"]), "golden rows")


# -------------------------------------------------- the workloads at full size

def nan_outputs(dev, o_shape, lse_shape):
    """Output buffers filled with NaN, so a row the kernels never write fails."""
    import torch
    o = torch.full(o_shape, float("nan"), dtype=torch.bfloat16, device=dev)
    lse = torch.full(lse_shape, float("nan"), dtype=torch.float32, device=dev)
    return o, lse


def run_fwd_nan(api, dev, data, scale, causal):
    import torch
    q, k, v = (to_dev(data[n], dev) for n in "qkv")
    B, Sq, Hq, _ = q.shape
    o, lse = nan_outputs(dev, q.shape, (B, Hq, Sq))
    api.attn_fwd(q, k, v, o=o, lse=lse, scale=scale, causal=causal)
    torch.cuda.synchronize()
    o, lse = bf16_to_np(o), f32_to_np(lse)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse)), "rows left unwritten"
    return o, lse


def item_rows(B, Hq, Sq, tile, seed):
    """One random row from every (batch, head, query tile of `tile` rows) work item."""
    rng = np.random.default_rng(seed)
    rows = []
    for b in range(B):
        for h in range(Hq):
            for t0 in range(0, Sq, tile):
                rows.append((b, h, int(rng.integers(t0, min(Sq, t0 + tile)))))
    return np.array(rows, dtype=np.int64)


def test_causal_prefill_workload_every_row(api, dev):
    """Workload 2 (B4 H16 S2048 d128, causal) in the benchmark's launch
    configuration, every output row against the C oracle (outputs start as
    NaN, so a work item the persistent walk skipped would fail)."""
    spec, data = si.make_workload("causal_prefill")
    o, lse = run_fwd_nan(api, dev, data, spec["scale"], True)
    o_ref, lse_ref = cpu.attn_full(data["q"], data["k"], data["v"], spec["scale"], True)
    err = assert_close(o, o_ref, lse, lse_ref, "workload 2, every row")
    print("workload 2 every row: max|dO| %.4g max|dLSE| %.3g" % err, flush=True)
    v = si.bf16_to_f64(data["v"])
    np.testing.assert_array_equal(o[:, 0], v[:, 0, :, :].repeat(spec["Hq"] // spec["Hkv"], axis=1))


def test_long_causal_workload_whole_heads_and_every_item(api, dev):
    """Workload 3 (B1 H32 S16384 d128, K of each head scaled by U(0.5, 2)):
    four whole heads (the sharpest and flattest K scales and two others) and
    one row of every 256-row work item of every head, against the C oracle."""
    spec, data = si.make_workload("long_causal")
    o, lse = run_fwd_nan(api, dev, data, spec["scale"], True)
    c = data["k_head_scale"]
    heads = sorted({int(np.argmax(c)), int(np.argmin(c)), 0, spec["Hq"] - 1})
    S = spec["Sq"]
    whole = np.array([(0, h, i) for h in heads for i in range(S)], dtype=np.int64)
    rows = np.concatenate([whole, item_rows(1, spec["Hq"], S, 256, seed=3)])
    o_ref, lse_ref = cpu.attn_rows(data["q"], data["k"], data["v"], spec["scale"], True, rows)
    b, h, i = rows[:, 0], rows[:, 1], rows[:, 2]
    err = assert_close(o[b, i, h], o_ref, lse[b, h, i], lse_ref, "workload 3")
    print("workload 3 heads %s (K scales %s) + every item: max|dO| %.4g max|dLSE| %.3g"
          % (heads, np.round(c[heads], 3).tolist(), *err), flush=True)


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_small_grid_long_items_sampled_rows(api, dev, causal):
    """B1 H8 S4096 d128: 128 items of 256 rows, fewer than the CUs, so the
    library runs 128-row items on 4-wave workgroups; each item walks up to
    64 key tiles.  One row of every 128-row item, tile edges and random rows
    against the oracle."""
    B, H, S, d = 1, 8, 4096, 128
    data = si.make_prefill(46, B, H, H, S, S, d)
    scale = si.default_scale(d)
    o, lse = run_fwd_nan(api, dev, data, scale, causal)
    rows = np.concatenate([sample_rows(B, H, S, 160, seed=46,
                                       extra_rows=(127, 128, 255, 256, 4095 - 128, 4095)),
                           item_rows(B, H, S, 128, seed=47)])
    o_ref, lse_ref = cpu.attn_rows(data["q"], data["k"], data["v"], scale, causal, rows)
    b, h, i = rows[:, 0], rows[:, 1], rows[:, 2]
    assert_close(o[b, i, h], o_ref, lse[b, h, i], lse_ref, "B1 H8 S4096")


@pytest.mark.parametrize("splits", [8, 0], ids=["8chunks_merge_kernel", "library_choice"])
def test_decode_workload_whole(api, dev, splits):
    """Workload 4 (B64 Hq32 Hkv8 Skv4096 d128) in full: with the 8 chunks of
    its recipe (split kernel, then the merge kernel over the partials) and
    with the library's choice (whole sequences per workgroup, no workspace)."""
    import torch
    spec, data = si.make_workload("gqa_decode")
    q, k, v = (to_dev(data[x], dev) for x in "qkv")
    o, lse = nan_outputs(dev, q.shape, q.shape[:2])
    B, Hq, Hkv, Skv, d = (spec[x] for x in ("B", "Hq", "Hkv", "Skv", "d"))
    assert (api.attn_decode_workspace_bytes(B, Hq, Hkv, Skv, d, splits) == 0) == (splits == 0)
    api.attn_decode(q, k, v, o=o, lse=lse, scale=spec["scale"], num_splits=splits)
    torch.cuda.synchronize()
    o_ref, lse_ref = cpu.decode_full(data["q"], data["k"], data["v"], spec["scale"])
    err = assert_close(bf16_to_np(o), o_ref, f32_to_np(lse), lse_ref, "workload 4")
    print("workload 4 (num_splits=%d): max|dO| %.4g max|dLSE| %.3g" % (splits, *err), flush=True)


def test_varlen_workload_two_heads_and_every_item(api, dev):
    """Workload 5 (16 ragged sequences, H32 d128, causal): every row of two
    heads across all 16 sequences, and one row of every (sequence, head,
    256-row tile) work item, against the C oracle; outputs start as NaN."""
    import torch
    spec, data = si.make_workload("ragged")
    cu = data["cu_seqlens"]
    maxlen = api.attn_varlen_check(cu, int(cu[-1]))
    q, k, v = (to_dev(data[x], dev) for x in "qkv")
    cu_d = torch.from_numpy(cu).to(dev)
    o, lse = nan_outputs(dev, q.shape, (spec["H"], q.shape[0]))
    api.attn_fwd_varlen(q, k, v, cu_d, cu_d, maxlen, maxlen, o=o, lse=lse, scale=spec["scale"],
                        causal=True)
    torch.cuda.synchronize()
    o, lse = bf16_to_np(o), f32_to_np(lse)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse)), "rows left unwritten"
    rng = np.random.default_rng(5)
    H = spec["H"]
    rows = []
    for s in range(spec["nseq"]):
        L = int(cu[s + 1] - cu[s])
        for h in (3, H - 5):
            rows.extend((s, h, i) for i in range(L))
        for h in range(H):
            for t0 in range(0, L, 256):
                rows.append((s, h, int(rng.integers(t0, min(L, t0 + 256)))))
    rows = np.array(rows, dtype=np.int64)
    o_ref, lse_ref = cpu.varlen_rows(data["q"], data["k"], data["v"], cu, cu, spec["scale"],
                                     True, rows)
    gi = cu[rows[:, 0]] + rows[:, 2]
    err = assert_close(o[gi, rows[:, 1]], o_ref, lse[rows[:, 1], gi], lse_ref, "workload 5")
    print("workload 5 two heads + every item: max|dO| %.4g max|dLSE| %.3g" % err, flush=True)


# -------------------------------------------------------------------- decode

DECODE = [  # B, Hq, Hkv, Skv, d, splits
    (2, 8, 2, 1000, 128, 7),
    (3, 4, 4, 1, 64, 1),
    (3, 4, 4, 1, 64, 4),            # more chunks than keys: empty chunks
    (1, 64, 1, 300, 128, 3),        # MQA group of 64 query heads (two column blocks)
    (2, 32, 8, 4096, 128, 0),       # library picks the split count
    (1, 40, 8, 513, 64, 2),
    (4, 16, 2, 129, 128, 1),
    # 256 or more (sequence, KV head) groups: an explicit split count is
    # honoured (split kernel, then the merge kernel), while 0 or 1 gives
    # whole sequences per workgroup, merged in the kernel (uneven last chunk;
    # chunks shorter than the load ring; empty chunks; d = 64)
    (64, 8, 4, 1000, 128, 7),
    (64, 8, 4, 1000, 128, 0),
    (64, 8, 4, 200, 128, 3),
    (64, 8, 4, 200, 128, 1),
    (32, 16, 8, 100, 128, 64),
    (128, 4, 2, 777, 64, 3),
    (128, 4, 2, 777, 64, 0),
    # few groups, many chunks: the merge kernel's unrolled loop and its tail
    (1, 32, 8, 5000, 128, 37),
    (2, 8, 2, 3000, 64, 100),       # six trailing chunks empty
]


@pytest.mark.parametrize("case", DECODE, ids=lambda c: "B%d_Hq%d_Hkv%d_Skv%d_d%d_s%d" % c)
def test_decode_matches_oracle(api, dev, case):
    import torch
    B, Hq, Hkv, Skv, d, splits = case
    data = si.make_decode(7 + Skv, B, Hq, Hkv, Skv, d)
    scale = si.default_scale(d)
    q, k, v = (to_dev(data[x], dev) for x in "qkv")
    o, lse = api.attn_decode(q, k, v, scale=scale, num_splits=splits)
    torch.cuda.synchronize()
    o_ref, lse_ref = cpu.decode_full(data["q"], data["k"], data["v"], scale)
    assert_close(bf16_to_np(o), o_ref, f32_to_np(lse), lse_ref, str(case))


DECODE_VARLEN = [  # B, Hq, Hkv, Skv_max, d, splits, lengths (None: random in [0, Skv_max])
    (4, 8, 2, 1000, 128, 7, [1000, 1, 0, 513]),
    (3, 4, 4, 300, 64, 1, [300, 17, 64]),
    (5, 16, 4, 777, 128, 0, None),
    (2, 64, 1, 200, 128, 3, [5, 200]),              # MQA, two column blocks
    (64, 8, 4, 1000, 128, 8, None),                  # groups fill the GPU: in-kernel merge
    (4, 8, 2, 256, 128, 4, [-5, 300, 256, 64]),      # out-of-range lengths are clamped
]


_decode_varlen_ref = decode_varlen_ref


@pytest.mark.parametrize("case", DECODE_VARLEN,
                         ids=lambda c: "B%d_Hq%d_Hkv%d_Skv%d_d%d_s%d" % c[:6])
def test_decode_varlen_matches_oracle(api, dev, case):
    """Per-sequence cache lengths (0, 1, full, random; clamped when out of range)."""
    import torch
    B, Hq, Hkv, Skv, d, splits, lengths = case
    data = si.make_decode(31 + Skv, B, Hq, Hkv, Skv, d)
    if lengths is None:
        lengths = np.random.default_rng(B + Skv).integers(0, Skv + 1, B)
    lengths = np.asarray(lengths, dtype=np.int32)
    scale = si.default_scale(d)
    q, k, v = (to_dev(data[x], dev) for x in "qkv")
    seq = torch.from_numpy(lengths).to(dev)
    o, lse = api.attn_decode_varlen(q, k, v, seq, scale=scale, num_splits=splits)
    torch.cuda.synchronize()
    o_ref, lse_ref = _decode_varlen_ref(data, np.clip(lengths, 0, Skv), scale)
    assert_close(bf16_to_np(o), o_ref, f32_to_np(lse), lse_ref, str(case[:6]))


def test_decode_varlen_full_lengths_equal_decode(api, dev):
    """Every sequence at full length: the same bits as attn_decode."""
    import torch
    for B, splits in ((4, 5), (64, 8)):
        data = si.make_decode(41, B, 16, 4, 640, 128)
        q, k, v = (to_dev(data[x], dev) for x in "qkv")
        seq = torch.full((B,), 640, dtype=torch.int32, device=dev)
        o1, l1 = api.attn_decode(q, k, v, num_splits=splits)
        o2, l2 = api.attn_decode_varlen(q, k, v, seq, num_splits=splits)
        torch.cuda.synchronize()
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
        assert torch.equal(l1, l2)


DECODE_PAGED = [  # B, Hq, Hkv, d, page_size, max_pages, splits, lengths (None: random)
    (4, 8, 2, 128, 16, 40, 4, [640, 1, 0, 333]),     # 16-key pages: a tile spans two pages
    (3, 16, 4, 128, 32, 10, 1, [320, 31, 200]),
    (5, 8, 8, 64, 64, 6, 0, None),
    (2, 32, 4, 128, 256, 4, 3, [1024, 700]),
    (64, 8, 2, 128, 128, 4, 8, None),                 # groups fill the GPU: whole sequences
    (3, 4, 1, 128, 48, 7, 2, [336, 47, 100]),         # page size a multiple of 16, not of 32
    (6, 16, 4, 128, 32, 64, 0, [2048, 100, 0, 1500, 33, 2047]),   # split by the lengths
]


@pytest.mark.parametrize("case", DECODE_PAGED,
                         ids=lambda c: "B%d_Hq%d_Hkv%d_d%d_page%d_x%d_s%d" % c[:7])
def test_decode_paged_matches_oracle(api, dev, case):
    """Paged cache with shuffled pages: same as the oracle on the gathered cache."""
    import torch
    B, Hq, Hkv, d, page, maxp, splits, lengths = case
    cap = page * maxp
    data = si.make_paged(77 + page + B, B, Hq, Hkv, d, page, maxp, B * maxp + 3)
    if lengths is None:
        lengths = np.random.default_rng(B + page).integers(0, cap + 1, B)
    lengths = np.asarray(lengths, dtype=np.int32)
    scale = si.default_scale(d)
    q = to_dev(data["q"], dev)
    kp, vp = to_dev(data["k_pages"], dev), to_dev(data["v_pages"], dev)
    table = torch.from_numpy(data["block_table"]).to(dev)
    seq = torch.from_numpy(lengths).to(dev)
    print("paged decode case", case[:7], flush=True)
    o, lse = api.attn_decode_paged(q, kp, vp, table, seq, scale=scale, num_splits=splits)
    torch.cuda.synchronize()
    dense = dict(q=data["q"], k=si.gather_pages(data["k_pages"], data["block_table"]),
                 v=si.gather_pages(data["v_pages"], data["block_table"]))
    o_ref, lse_ref = _decode_varlen_ref(dense, np.clip(lengths, 0, cap), scale)
    assert_close(bf16_to_np(o), o_ref, f32_to_np(lse), lse_ref, str(case[:7]))


def test_decode_paged_identity_table_equals_varlen(api, dev):
    """Pages laid out in order (page id = b * max_pages + i): the same bits as
    decode over the equivalent dense cache."""
    import torch
    B, Hq, Hkv, d, page, maxp = 6, 16, 4, 128, 64, 8
    data = si.make_decode(43, B, Hq, Hkv, page * maxp, d)
    lengths = torch.tensor([512, 1, 0, 300, 64, 129], dtype=torch.int32, device=dev)
    q, k, v = (to_dev(data[x], dev) for x in "qkv")
    kp = k.reshape(B * maxp, page, Hkv, d)
    vp = v.reshape(B * maxp, page, Hkv, d)
    table = torch.arange(B * maxp, dtype=torch.int32, device=dev).reshape(B, maxp)
    for splits in (1, 4):
        o1, l1 = api.attn_decode_varlen(q, k, v, lengths, num_splits=splits)
        o2, l2 = api.attn_decode_paged(q, kp, vp, table, lengths, num_splits=splits)
        torch.cuda.synchronize()
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
        assert torch.equal(l1, l2)


DECODE_FP8 = [  # B, Hq, Hkv, Skv, d, splits, lengths (None: every key; "rand": random)
    (2, 8, 2, 1000, 128, 7, None),
    (3, 4, 4, 1, 64, 1, None),
    (3, 4, 4, 1, 64, 4, None),                 # more chunks than keys: empty chunks
    (1, 64, 1, 300, 128, 3, None),             # MQA group of 64 query heads
    (2, 32, 8, 4096, 128, 0, None),            # library picks the split count
    (1, 40, 8, 513, 64, 2, None),
    (4, 16, 2, 129, 128, 1, None),             # one chunk, ragged last 64-key tile
    (64, 8, 4, 1000, 128, 7, None),            # groups fill the GPU: in-kernel merge
    (128, 4, 2, 777, 64, 3, None),
    (4, 8, 2, 1000, 128, 7, [1000, 1, 0, 513]),
    (5, 16, 4, 777, 128, 0, "rand"),
    (64, 8, 4, 1000, 128, 8, "rand"),
    (4, 8, 2, 256, 128, 4, [-5, 300, 256, 64]),   # out-of-range lengths are clamped
]


def _run_decode_fp8(api, dev, data, scale, splits, lengths=None):
    import torch
    q = to_dev(data["q"], dev)
    k = torch.from_numpy(data["k"]).to(dev)
    v = torch.from_numpy(data["v"]).to(dev)
    seq = None if lengths is None else torch.from_numpy(np.asarray(lengths, np.int32)).to(dev)
    o, lse = api.attn_decode_fp8(q, k, v, data["k_scale"], data["v_scale"], seqlens_k=seq,
                                 scale=scale, num_splits=splits)
    torch.cuda.synchronize()
    return bf16_to_np(o), f32_to_np(lse)


@pytest.mark.parametrize("case", DECODE_FP8, ids=lambda c: "B%d_Hq%d_Hkv%d_Skv%d_d%d_s%d" % c[:6])
def test_decode_fp8_matches_oracle(api, dev, case):
    """fp8 (e4m3fn) caches with per-tensor scales against the oracle's dequantised decode."""
    B, Hq, Hkv, Skv, d, splits, lengths = case
    data = si.make_decode_fp8(41 + Skv, B, Hq, Hkv, Skv, d)
    if isinstance(lengths, str):
        lengths = np.random.default_rng(B + Skv).integers(0, Skv + 1, B)
    scale = si.default_scale(d)
    o, lse = _run_decode_fp8(api, dev, data, scale, splits, lengths)
    o_ref, lse_ref = ref.decode_fp8(si.bf16_to_f64(data["q"]), data["k"], data["v"], scale,
                                    data["k_scale"], data["v_scale"], seqlens=lengths)
    assert_close(o, o_ref, lse, lse_ref, str(case[:6]))


def test_decode_fp8_workload_sampled_sequences(api, dev):
    """The decode workload's sizes (B64 Hq32 Hkv8 Skv4096 d128, 8 chunks) with an fp8
    cache, in the launch configuration the benchmark times; the oracle checks
    eight whole sequences."""
    spec = si.WORKLOADS["gqa_decode"]
    B, Hq, Hkv, Skv, d = (spec[x] for x in ("B", "Hq", "Hkv", "Skv", "d"))
    data = si.make_decode_fp8(spec["seed"], B, Hq, Hkv, Skv, d)
    scale = si.default_scale(d)
    o, lse = _run_decode_fp8(api, dev, data, scale, spec["num_splits"])
    bs = np.array([0, 1, 17, 31, 32, 50, 62, 63])
    o_ref, lse_ref = ref.decode_fp8(si.bf16_to_f64(data["q"][bs]), data["k"][bs], data["v"][bs],
                                    scale, data["k_scale"], data["v_scale"])
    assert_close(o[bs], o_ref, lse[bs], lse_ref, "fp8 decode workload")
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))


def test_decode_fp8_power_of_two_scales_equal_bf16_cache(api, dev):
    """Codes times a power-of-two scale are exact bf16 values, so the bf16 decode of
    that cache computes the same attention; the two paths agree to rounding."""
    import torch
    B, Hq, Hkv, Skv, d = 4, 16, 4, 900, 128
    data = si.make_decode_fp8(77, B, Hq, Hkv, Skv, d)
    data["k_scale"], data["v_scale"] = 2.0 ** -6, 2.0 ** -7
    o8, l8 = _run_decode_fp8(api, dev, data, 0.09, 3)
    kb = torch.from_numpy(data["k"]).view(torch.float8_e4m3fn).to(torch.float32) * 2.0 ** -6
    vb = torch.from_numpy(data["v"]).view(torch.float8_e4m3fn).to(torch.float32) * 2.0 ** -7
    q = to_dev(data["q"], dev)
    o16, l16 = api.attn_decode(q, kb.to(torch.bfloat16).to(dev), vb.to(torch.bfloat16).to(dev),
                               scale=0.09, num_splits=3)
    torch.cuda.synchronize()
    assert np.abs(o8 - bf16_to_np(o16)).max() <= 2 ** -6
    assert np.abs(l8 - f32_to_np(l16)).max() <= 1e-4


def test_decode_workspace_reused_across_shapes(api, dev):
    """One workspace (uninitialised) serves successive split decodes of
    different shapes: nothing in it carries over from one call to the next."""
    import torch
    cases = [(1, 32, 8, 5000, 128, 37), (3, 16, 4, 3000, 64, 9), (2, 8, 2, 9000, 128, 64),
             (1, 32, 8, 5000, 128, 37)]
    need = max(api.attn_decode_workspace_bytes(B, Hq, Hkv, S, d, s) for B, Hq, Hkv, S, d, s in cases)
    ws = torch.full((need,), 0x7F, dtype=torch.uint8, device=dev)
    for B, Hq, Hkv, Skv, d, splits in cases:
        data = si.make_decode(90 + Skv, B, Hq, Hkv, Skv, d)
        q, k, v = (to_dev(data[x], dev) for x in "qkv")
        o, lse = api.attn_decode(q, k, v, num_splits=splits, workspace=ws)
        torch.cuda.synchronize()
        o_ref, lse_ref = cpu.decode_full(data["q"], data["k"], data["v"], si.default_scale(d))
        assert_close(bf16_to_np(o), o_ref, f32_to_np(lse), lse_ref, str((B, Hq, Hkv, Skv, d, splits)))


def test_decode_split_counts_agree(api, dev):
    """1, 2, 8, 64 chunks and the library's choice agree closely (fp32 merge)."""
    import torch
    data = si.make_decode(11, 4, 16, 4, 2048, 128)
    q, k, v = (to_dev(data[x], dev) for x in "qkv")
    outs = []
    for s in (1, 2, 8, 64, 0):
        o, lse = api.attn_decode(q, k, v, num_splits=s)
        torch.cuda.synchronize()
        outs.append((bf16_to_np(o), f32_to_np(lse)))
    for o, lse in outs[1:]:
        assert np.abs(o - outs[0][0]).max() <= 2 ** -6
        assert np.abs(lse - outs[0][1]).max() <= 2e-5


def test_decode_equals_prefill_last_row(api, dev):
    """Decode of the newest token == the last row of a causal prefill."""
    import torch
    B, Hq, Hkv, S, d = 2, 8, 2, 700, 128
    data = si.make_prefill(12, B, Hq, Hkv, S, S, d)
    q, k, v = (to_dev(data[x], dev) for x in "qkv")
    o_p, l_p = api.attn_fwd(q, k, v, causal=True)
    o_d, l_d = api.attn_decode(q[:, -1].contiguous(), k, v, num_splits=3)
    torch.cuda.synchronize()
    assert np.abs(bf16_to_np(o_d) - bf16_to_np(o_p[:, -1])).max() <= 2 ** -6
    assert np.abs(f32_to_np(l_d) - f32_to_np(l_p[:, :, -1])).max() <= 1e-4


# ---------------------------------------------------- split-KV prefill

SPLITKV = [  # B, Sq, Skv, Hq, Hkv, d, causal, splits
    (1, 512, 8192, 32, 8, 128, True, 4),      # a chunk of new tokens against a long cache
    (2, 300, 300, 4, 4, 64, True, 3),         # ragged tile ends, d = 64
    (1, 1000, 1000, 8, 2, 128, False, 0),     # library's choice, non-causal GQA
    (1, 256, 256, 2, 2, 64, True, 8),         # more shares than key tiles: empty shares
    (3, 100, 5000, 4, 4, 128, True, 16),      # one partial query tile per head
    (1, 1024, 1024, 32, 32, 128, True, 0),    # few query tiles, library's choice
]


@pytest.mark.parametrize("case", SPLITKV, ids=lambda c: "B%d_Sq%d_Skv%d_Hq%d_Hkv%d_d%d_%s_s%d" % (
    c[0], c[1], c[2], c[3], c[4], c[5], "causal" if c[6] else "full", c[7]))
def test_fwd_splitkv_matches_oracle(api, dev, case):
    import torch
    B, Sq, Skv, Hq, Hkv, d, causal, splits = case
    data = si.make_prefill(60 + Sq + Skv, B, Hq, Hkv, Sq, Skv, d)
    scale = si.default_scale(d)
    q, k, v = (to_dev(data[n], dev) for n in "qkv")
    o, lse = api.attn_fwd_splitkv(q, k, v, scale=scale, causal=causal, num_splits=splits)
    torch.cuda.synchronize()
    o_ref, lse_ref = cpu.attn_full(data["q"], data["k"], data["v"], scale, causal)
    assert_close(bf16_to_np(o), o_ref, f32_to_np(lse), lse_ref, str(case))


def test_fwd_splitkv_one_split_is_attn_fwd_bitwise(api, dev):
    import torch
    data = si.make_prefill(71, 2, 8, 4, 700, 700, 128)
    q, k, v = (to_dev(data[n], dev) for n in "qkv")
    o1, l1 = api.attn_fwd(q, k, v, causal=True)
    o2, l2 = api.attn_fwd_splitkv(q, k, v, causal=True, num_splits=1)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


def test_fwd_splitkv_split_counts_agree(api, dev):
    """2, 5 and 13 shares agree with the unsplit forward to fp32 merge rounding."""
    import torch
    data = si.make_prefill(72, 1, 16, 4, 640, 4000, 128)
    q, k, v = (to_dev(data[n], dev) for n in "qkv")
    o1, l1 = api.attn_fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    for s in (2, 5, 13):
        o2, l2 = api.attn_fwd_splitkv(q, k, v, causal=True, num_splits=s)
        torch.cuda.synchronize()
        assert np.abs(bf16_to_np(o2) - bf16_to_np(o1)).max() <= 2 ** -6, s
        assert np.abs(f32_to_np(l2) - f32_to_np(l1)).max() <= 1e-4, s


# ------------------------------------------------- invariants and equivalences

def test_constant_v_gives_the_constant(api, dev):
    """V rows all equal to a bf16 vector c: every output row is c to one bf16 ulp.

    The weights enter the second product rounded to bf16 while the row sum
    adds them unrounded, so sum(P)/l differs from 1 by at most 2^-9.
    """
    import torch
    B, S, H, d = 2, 300, 4, 128
    data = si.make_prefill(13, B, H, H, S, S, d)
    c = data["v"][0, 0, 0].copy()
    data["v"][:] = c
    for causal in (False, True):
        o, _ = run_fwd(api, dev, data, si.default_scale(d), causal)
        np.testing.assert_allclose(o, np.broadcast_to(si.bf16_to_f64(c), o.shape), rtol=2 ** -7,
                                   atol=0)
    q, k, v = (to_dev(data[x], dev) for x in "qkv")
    od, _ = api.attn_decode(q[:, -1].contiguous(), k, v, num_splits=5)
    torch.cuda.synchronize()
    np.testing.assert_allclose(bf16_to_np(od), np.broadcast_to(si.bf16_to_f64(c), od.shape),
                               rtol=2 ** -7, atol=0)


def test_zero_query_gives_mean_and_log_count(api, dev):
    B, S, H, d = 1, 260, 2, 64
    data = si.make_prefill(14, B, H, H, S, S, d)
    data["q"][:] = 0
    o, lse = run_fwd(api, dev, data, 0.125, True)
    v = si.bf16_to_f64(data["v"])
    mean = np.cumsum(v, axis=1) / np.arange(1, S + 1)[None, :, None, None]
    assert np.abs(o - mean).max() <= 2e-2
    np.testing.assert_allclose(lse, np.broadcast_to(np.log(np.arange(1, S + 1)), lse.shape),
                               atol=1e-4)


def test_large_scores_do_not_overflow(api, dev):
    """Scores of several hundred in scaled units: finite and equal to the oracle."""
    B, S, H, d = 1, 256, 2, 128
    data = si.make_prefill(15, B, H, H, S, S, d)
    q = si.bf16_to_f32(data["q"]) * 8.0
    data["q"] = si.f32_to_bf16_bits(q)
    o, lse = run_fwd(api, dev, data, 1.0, True)
    o_ref, lse_ref = cpu.attn_full(data["q"], data["k"], data["v"], 1.0, True)
    assert lse_ref.max() > 300
    assert_close(o, o_ref, lse, lse_ref, "large scores")


def test_bitwise_deterministic(api, dev):
    spec = si.WORKLOADS["causal_prefill"]
    data = si.make_prefill(16, 2, 8, 8, 1024, 1024, 128)
    a = run_fwd(api, dev, data, 0.088, True)
    for _ in range(3):
        b = run_fwd(api, dev, data, 0.088, True)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_gqa_equals_repeated_mha_bitwise(api, dev):
    B, S, Hq, Hkv, d = 2, 320, 8, 2, 128
    data = si.make_prefill(17, B, Hq, Hkv, S, S, d)
    rep = dict(q=data["q"], k=np.repeat(data["k"], 4, axis=2), v=np.repeat(data["v"], 4, axis=2))
    for causal in (False, True):
        a = run_fwd(api, dev, data, 0.09, causal)
        b = run_fwd(api, dev, rep, 0.09, causal)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_varlen_equals_separate_calls_bitwise(api, dev):
    import torch
    lengths = [1, 130, 7, 300, 128]
    data = si.make_varlen(18, len(lengths), 1, 300, H=4, d=128, Hkv=2, lengths=lengths)
    cu = data["cu_seqlens"]
    q, k, v = (to_dev(data[x], dev) for x in "qkv")
    cu_d = torch.from_numpy(cu).to(dev)
    for causal in (False, True):
        o, lse = api.attn_fwd_varlen(q, k, v, cu_d, cu_d, max(lengths), max(lengths),
                                     scale=0.09, causal=causal)
        torch.cuda.synchronize()
        o, lse = bf16_to_np(o), f32_to_np(lse)
        for s, L in enumerate(lengths):
            a, b = cu[s], cu[s + 1]
            sub = {x: data[x][a:b][None] for x in "qkv"}
            os_, ls_ = run_fwd(api, dev, sub, 0.09, causal)
            assert np.array_equal(o[a:b], os_[0]) and np.array_equal(lse[:, a:b], ls_[0])


VARLEN_CROSS = [  # d, Hq, Hkv, query lengths, key lengths (chunked prefill, empty sides)
    (128, 4, 2, [5, 0, 300, 64, 1, 200], [100, 7, 300, 0, 400, 77]),
    (64, 6, 3, [129, 3, 0, 130], [1000, 3, 1, 129]),
]


@pytest.mark.parametrize("case", VARLEN_CROSS, ids=["d128", "d64"])
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_varlen_cross_lengths_match_oracle(api, dev, case, causal):
    """Query and key lengths differ per sequence, either may be 0.

    Every query row is compared with the oracle; rows of a sequence with no
    keys (and, under the bottom-right causal mask, leading rows of a sequence
    with more queries than keys) must be exactly O = 0, LSE = -inf.
    """
    import torch
    d, Hq, Hkv, lq, lk = case
    data = si.make_varlen_cross(21 + d, lq, lk, H=Hq, d=d, Hkv=Hkv)
    cq, ck = data["cu_seqlens_q"], data["cu_seqlens_k"]
    q, k, v = (to_dev(data[x], dev) for x in "qkv")
    cq_d, ck_d = torch.from_numpy(cq).to(dev), torch.from_numpy(ck).to(dev)
    scale = si.default_scale(d)
    print("varlen cross d=%d causal=%d lq=%s lk=%s" % (d, causal, lq, lk), flush=True)
    o, lse = api.attn_fwd_varlen(q, k, v, cq_d, ck_d, max(lq), max(lk), scale=scale,
                                 causal=causal)
    torch.cuda.synchronize()
    o, lse = bf16_to_np(o), f32_to_np(lse)
    rows = np.array([(s, h, i) for s in range(len(lq)) for h in range(Hq) for i in range(lq[s])],
                    dtype=np.int64)
    o_ref, lse_ref = cpu.varlen_rows(data["q"], data["k"], data["v"], cq, ck, scale, causal, rows)
    tok = cq[rows[:, 0]] + rows[:, 2]
    assert_close(o[tok, rows[:, 1]], o_ref, lse[rows[:, 1], tok], lse_ref, str(case))
    for s in range(len(lq)):
        dead = lq[s] if lk[s] == 0 else (max(0, lq[s] - lk[s]) if causal else 0)
        a = cq[s]
        assert np.all(o[a:a + dead] == 0) and np.all(np.isneginf(lse[:, a:a + dead]))


# Ragged batches with at least as many (sequence, head, 256-row tile) items
# as compute units run on a persistent grid whose workgroups each list their
# items, cost-sorted, in LDS; up to 256 sequences and 1024 query tiles,
# beyond that in the launcher's own order.
def _compact_rows(rng, lq, Hq, heads=(0,), per_item=1):
    """Every row of the given heads, and per_item random rows of every
    (sequence, head, 256-row tile)."""
    rows = []
    for s, L in enumerate(lq):
        for h in heads:
            rows.extend((s, h, i) for i in range(L))
        for h in range(Hq):
            for t0 in range(0, L, 256):
                for _ in range(per_item):
                    rows.append((s, h, int(rng.integers(t0, min(L, t0 + 256)))))
    return np.array(rows, dtype=np.int64)


def test_varlen_listed_schedule_equals_separate_calls_bitwise(api, dev):
    """A ragged batch on the listed schedule (7 sequences x 32 heads x up to 8
    query tiles) gives bit for bit what one call per sequence gives."""
    import torch
    lengths = [1, 130, 7, 2000, 128, 513, 300]
    data = si.make_varlen(31, len(lengths), 1, 2000, H=32, d=128, Hkv=8, lengths=lengths)
    cu = data["cu_seqlens"]
    q, k, v = (to_dev(data[x], dev) for x in "qkv")
    cu_d = torch.from_numpy(cu).to(dev)
    for causal in (False, True):
        print("listed schedule vs separate calls, causal=%d" % causal, flush=True)
        o, lse = api.attn_fwd_varlen(q, k, v, cu_d, cu_d, max(lengths), max(lengths),
                                     scale=0.09, causal=causal)
        torch.cuda.synchronize()
        o, lse = bf16_to_np(o), f32_to_np(lse)
        for s, L in enumerate(lengths):
            a, b = cu[s], cu[s + 1]
            sub = {x: data[x][a:b][None] for x in "qkv"}
            os_, ls_ = run_fwd(api, dev, sub, 0.09, causal)
            assert np.array_equal(o[a:b], os_[0]) and np.array_equal(lse[:, a:b], ls_[0]), s


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_varlen_listed_schedule_cross_lengths(api, dev, causal):
    """The listed schedule with query and key lengths that differ (either may
    be 0, empty sequences included): sampled rows against the oracle; rows
    with no keys exactly O = 0, LSE = -inf; outputs start as NaN."""
    import torch
    rng = np.random.default_rng(77)
    n = 40
    lq = [int(x) for x in rng.integers(0, 700, n)]
    lk = [int(x) for x in rng.integers(0, 900, n)]
    lq[3], lk[5], lq[7], lk[7] = 0, 0, 0, 0
    lk[9] = lq[9] // 3                       # more queries than keys
    Hq, Hkv, d = 16, 4, 128
    data = si.make_varlen_cross(78, lq, lk, H=Hq, d=d, Hkv=Hkv)
    cq, ck = data["cu_seqlens_q"], data["cu_seqlens_k"]
    q, k, v = (to_dev(data[x], dev) for x in "qkv")
    o, lse = nan_outputs(dev, q.shape, (Hq, q.shape[0]))
    print("listed schedule cross lengths causal=%d" % causal, flush=True)
    api.attn_fwd_varlen(q, k, v, torch.from_numpy(cq).to(dev), torch.from_numpy(ck).to(dev),
                        max(lq), max(lk), o=o, lse=lse, scale=si.default_scale(d), causal=causal)
    torch.cuda.synchronize()
    o, lse = bf16_to_np(o), f32_to_np(lse)
    assert not np.isnan(o).any() and not np.isnan(lse).any(), "rows left unwritten"
    rows = _compact_rows(rng, lq, Hq, heads=(0, Hq - 1), per_item=2)
    o_ref, lse_ref = cpu.varlen_rows(data["q"], data["k"], data["v"], cq, ck,
                                     si.default_scale(d), causal, rows)
    tok = cq[rows[:, 0]] + rows[:, 2]
    assert_close(o[tok, rows[:, 1]], o_ref, lse[rows[:, 1], tok], lse_ref, "listed cross")
    for s in range(n):
        dead = lq[s] if lk[s] == 0 else (max(0, lq[s] - lk[s]) if causal else 0)
        a = cq[s]
        assert np.all(o[a:a + dead] == 0) and np.all(np.isneginf(lse[:, a:a + dead])), s


def test_varlen_more_sequences_than_the_list_holds(api, dev):
    """300 sequences (past the listed schedule's 256): the launcher's order on
    a persistent grid; sampled rows of every item against the oracle."""
    import torch
    rng = np.random.default_rng(79)
    lengths = [int(x) for x in rng.integers(1, 400, 300)]
    Hq, d = 4, 64
    data = si.make_varlen(80, len(lengths), 1, 400, H=Hq, d=d, Hkv=2, lengths=lengths)
    cu = data["cu_seqlens"]
    q, k, v = (to_dev(data[x], dev) for x in "qkv")
    o, lse = nan_outputs(dev, q.shape, (Hq, q.shape[0]))
    print("300 sequences, causal", flush=True)
    api.attn_fwd_varlen(q, k, v, torch.from_numpy(cu).to(dev), torch.from_numpy(cu).to(dev),
                        max(lengths), max(lengths), o=o, lse=lse, scale=si.default_scale(d),
                        causal=True)
    torch.cuda.synchronize()
    o, lse = bf16_to_np(o), f32_to_np(lse)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse)), "rows left unwritten"
    rows = _compact_rows(rng, lengths, Hq, heads=(1,), per_item=1)
    o_ref, lse_ref = cpu.varlen_rows(data["q"], data["k"], data["v"], cu, cu,
                                     si.default_scale(d), True, rows)
    gi = cu[rows[:, 0]] + rows[:, 2]
    assert_close(o[gi, rows[:, 1]], o_ref, lse[rows[:, 1], gi], lse_ref, "300 sequences")


def _varlen_sampled(api, dev, lengths, H, Hkv, d, seed, heads, per_item, label):
    """One causal ragged call (outputs start as NaN), every row of the given
    heads and per_item random rows of every (sequence, head, 256-row tile)
    against the oracle."""
    import torch
    rng = np.random.default_rng(seed)
    data = si.make_varlen(seed, len(lengths), 1, max(lengths), H=H, d=d, Hkv=Hkv, lengths=lengths)
    cu = data["cu_seqlens"]
    q, k, v = (to_dev(data[x], dev) for x in "qkv")
    o, lse = nan_outputs(dev, q.shape, (H, q.shape[0]))
    print(label, flush=True)
    api.attn_fwd_varlen(q, k, v, torch.from_numpy(cu).to(dev), torch.from_numpy(cu).to(dev),
                        max(lengths), max(lengths), o=o, lse=lse, scale=si.default_scale(d),
                        causal=True)
    torch.cuda.synchronize()
    o, lse = bf16_to_np(o), f32_to_np(lse)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse)), "rows left unwritten"
    rows = _compact_rows(rng, lengths, H, heads=heads, per_item=per_item)
    o_ref, lse_ref = cpu.varlen_rows(data["q"], data["k"], data["v"], cu, cu,
                                     si.default_scale(d), True, rows)
    gi = cu[rows[:, 0]] + rows[:, 2]
    return assert_close(o[gi, rows[:, 1]], o_ref, lse[rows[:, 1], gi], lse_ref, label)


def test_varlen_listed_schedule_at_its_bounds(api, dev):
    """256 sequences (the list's sequence bound), the longest 262,144 tokens
    (1024 query tiles: the level bound) and 1 head: 262,144 item slots, the
    launcher's bound for the list on 256 CUs (1024 per workgroup)."""
    rng = np.random.default_rng(81)
    lengths = [int(x) for x in rng.integers(1, 300, 256)]
    lengths[100] = 262144
    err = _varlen_sampled(api, dev, lengths, 1, 1, 64, 82, heads=(), per_item=1,
                          label="listed schedule at its bounds")
    print("max|dO| %.4g max|dLSE| %.3g" % err, flush=True)


def test_varlen_one_workgroup_per_item(api, dev):
    """257 sequences, some past 512 tokens: past the list's sequence bound and
    the short-sequence rule, so one workgroup per item."""
    rng = np.random.default_rng(83)
    lengths = [int(x) for x in rng.integers(1, 1200, 257)]
    err = _varlen_sampled(api, dev, lengths, 2, 1, 128, 84, heads=(1,), per_item=1,
                          label="one workgroup per item, 257 sequences")
    print("max|dO| %.4g max|dLSE| %.3g" % err, flush=True)


def test_lse_optional(api, dev):
    import torch
    data = si.make_prefill(19, 1, 2, 2, 200, 200, 64)
    q, k, v = (to_dev(data[x], dev) for x in "qkv")
    o1, _ = api.attn_fwd(q, k, v, causal=True)
    o2, l2 = api.attn_fwd(q, k, v, causal=True, want_lse=False)
    torch.cuda.synchronize()
    assert l2 is None and torch.equal(o1, o2)
