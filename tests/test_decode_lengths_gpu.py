"""GPU parity of the decode split by the per-sequence lengths.

With per-sequence key counts, the library's split choice (num_splits <= 0)
and a workspace of attn_decode_varlen_workspace_bytes, the split kernel lays
the 32-key tiles of every (sequence, KV head, query-head block) group end to
end and gives each of the 1024 waves of its grid an equal run of them; a
group inside one run gets its result directly, the merge kernel merges the
runs of the others.  Every case is checked against the fp64 oracle (O within
2e-2, LSE within 1e-3), and the header the kernel wrote into the workspace
against the documented rule: the run length ceil(tiles / 1024), at least 4,
and each sequence's first tile.
"""
import math

import numpy as np
import pytest

import synth_inputs as si
from oracle import ref
from tests.gpu_util import assert_close, bf16_to_np, decode_varlen_ref, f32_to_np, to_dev

pytestmark = pytest.mark.gpu

MIN_TILES = 4
WAVES = 1024
MAX_SEQS = 2048


@pytest.fixture(scope="module")
def api():
    from tiled_attention_transformer_amd import api as a
    a._lib.load()
    return a


def expected_header(lengths, Skv, Hq, Hkv):
    """(run length in tiles, first tile of every sequence and the total)."""
    L = np.clip(np.asarray(lengths, np.int64), 0, Skv)
    per = Hkv * math.ceil(Hq // Hkv / 32)
    offs = np.concatenate([[0], np.cumsum(-(-L // 32) * per)])
    return max(MIN_TILES, -(-int(offs[-1]) // WAVES)), offs.tolist()


def lengths_of(spec, B, Skv, seed):
    if isinstance(spec, str):
        rng = np.random.default_rng(seed)
        if spec == "rand":
            return rng.integers(0, Skv + 1, B).astype(np.int32)
        if spec == "skew":   # one full sequence among 256-key ones
            L = np.full(B, 256, np.int32)
            L[int(rng.integers(B))] = Skv
            return L
    return np.asarray(spec, np.int32)


def header(ws, B):
    import torch
    h = ws[:16 + 4 * (B + 1)].cpu().view(torch.int32).tolist()
    return h[0], h[4:]


def ws_bytes(B, Hq, Hkv, d):
    return 16 + -(-4 * (B + 1) // 16) * 16 + (B * Hq + WAVES * min(Hq // Hkv, 32)) * (d + 1) * 4


LISTED = [  # B, Hq, Hkv, Skv_max, d, lengths
    (32, 8, 2, 8192, 128, "skew"),
    (8, 16, 4, 3000, 128, [3000, 0, 1, 511, 512, 513, 2999, 0]),     # chunk edges, empty sequences
    (6, 8, 2, 2000, 64, [0] * 6),                                    # no keys at all: no items
    (16, 64, 1, 1500, 128, "rand"),                                  # MQA, two query-head blocks
    (4, 8, 8, 32768, 64, [32768, 30000, 17, 25000]),                 # chunk above the minimum
    (MAX_SEQS, 4, 1, 1024, 64, "rand"),                              # the longest list
    (12, 8, 2, 5000, 128, [300] * 12),                               # every group over several runs
    (1024, 8, 8, 64, 64, [32] * 1024),                               # 8 groups a run: no merge
    (2, 32, 8, 40000, 128, [40000, 1]),                              # few long groups: many runs each
    (32, 8, 8, 3000, 64, "rand"),                                    # 256 groups
    (300, 8, 2, 100, 128, "rand"),                                   # groups whole and split
    (3, 8, 2, 700, 128, [-7, 800, 650]),                             # out-of-range lengths clamped
]


@pytest.mark.parametrize("case", LISTED, ids=lambda c: "B%d_Hq%d_Hkv%d_Skv%d_d%d" % c[:5])
def test_length_split_matches_oracle(api, dev, case):
    import torch
    B, Hq, Hkv, Skv, d, spec = case
    lengths = lengths_of(spec, B, Skv, B + Skv)
    data = si.make_decode(500 + B + Skv, B, Hq, Hkv, Skv, d)
    scale = si.default_scale(d)
    q, k, v = (to_dev(data[x], dev) for x in "qkv")
    seq = torch.from_numpy(lengths).to(dev)
    need = api.attn_decode_varlen_workspace_bytes(B, Hq, Hkv, Skv, d)
    assert need == ws_bytes(B, Hq, Hkv, d)
    ws = torch.full((need,), 0x7F, dtype=torch.uint8, device=dev)
    print("length-split decode", case[:5], flush=True)
    o, lse = api.attn_decode_varlen(q, k, v, seq, scale=scale, num_splits=0, workspace=ws)
    torch.cuda.synchronize()
    assert header(ws, B) == expected_header(lengths, Skv, Hq, Hkv)
    o_ref, lse_ref = decode_varlen_ref(data, np.clip(lengths, 0, Skv), scale)
    assert_close(bf16_to_np(o), o_ref, f32_to_np(lse), lse_ref, str(case[:5]))


def test_length_split_agrees_with_capacity_split(api, dev):
    """The split by the lengths and by the capacity (an explicit count, and the
    library's choice with the smaller workspace) agree to fp32 merge rounding."""
    import torch
    B, Hq, Hkv, Skv, d = 24, 16, 4, 4096, 128
    lengths = lengths_of("rand", B, Skv, 5)
    data = si.make_decode(61, B, Hq, Hkv, Skv, d)
    q, k, v = (to_dev(data[x], dev) for x in "qkv")
    seq = torch.from_numpy(lengths).to(dev)
    small = api.attn_decode_workspace_bytes(B, Hq, Hkv, Skv, d, 0)
    ws_small = torch.empty(max(small, 16), dtype=torch.uint8, device=dev)
    runs = [api.attn_decode_varlen(q, k, v, seq, num_splits=0),
            api.attn_decode_varlen(q, k, v, seq, num_splits=8),
            api.attn_decode_varlen(q, k, v, seq, num_splits=0, workspace=ws_small)]
    torch.cuda.synchronize()
    outs = [(bf16_to_np(o), f32_to_np(l)) for o, l in runs]
    for o, l in outs[1:]:
        assert np.abs(o - outs[0][0]).max() <= 2 ** -6
        fin = np.isfinite(outs[0][1])
        assert np.array_equal(fin, np.isfinite(l))
        assert np.abs(l[fin] - outs[0][1][fin]).max() <= 2e-5


def test_length_split_workspace_reused(api, dev):
    """One dirty workspace serves successive calls whose lengths give
    different run lengths (the header is rewritten by every call)."""
    import torch
    B, Hq, Hkv, Skv, d = 8, 8, 4, 32768, 64       # runs of 32, 5 and 4 tiles
    data = si.make_decode(71, B, Hq, Hkv, Skv, d)
    scale = si.default_scale(d)
    q, k, v = (to_dev(data[x], dev) for x in "qkv")
    ws = torch.full((api.attn_decode_varlen_workspace_bytes(B, Hq, Hkv, Skv, d),), 0x55,
                    dtype=torch.uint8, device=dev)
    chunks = set()
    for spec in ([Skv] * B, "skew", [40] * B, "rand"):
        lengths = lengths_of(spec, B, Skv, 9)
        o, lse = api.attn_decode_varlen(q, k, v, torch.from_numpy(lengths).to(dev),
                                        scale=scale, workspace=ws)
        torch.cuda.synchronize()
        hdr = header(ws, B)
        assert hdr == expected_header(lengths, Skv, Hq, Hkv)
        chunks.add(hdr[0])
        o_ref, lse_ref = decode_varlen_ref(data, np.clip(lengths, 0, Skv), scale)
        assert_close(bf16_to_np(o), o_ref, f32_to_np(lse), lse_ref, str(spec)[:40])
    assert len(chunks) == 4       # 32, 5, 4 and 19 tiles


def test_more_sequences_than_the_list_split_by_capacity(api, dev):
    """Past the list's 2048 sequences the call splits by the capacity (the
    sizing helper says so) and is still exact."""
    import torch
    B, Hq, Hkv, Skv, d = MAX_SEQS + 1, 4, 1, 600, 64
    assert api.attn_decode_varlen_workspace_bytes(B, Hq, Hkv, Skv, d) == \
        api.attn_decode_workspace_bytes(B, Hq, Hkv, Skv, d, 0)
    lengths = lengths_of("rand", B, Skv, 3)
    data = si.make_decode(81, B, Hq, Hkv, Skv, d)
    scale = si.default_scale(d)
    q, k, v = (to_dev(data[x], dev) for x in "qkv")
    o, lse = api.attn_decode_varlen(q, k, v, torch.from_numpy(lengths).to(dev), scale=scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = decode_varlen_ref(data, lengths, scale)
    assert_close(bf16_to_np(o), o_ref, f32_to_np(lse), lse_ref, "B2049")


FP8 = [  # B, Hq, Hkv, Skv, d, lengths
    (32, 8, 2, 8192, 128, "skew"),
    (8, 16, 4, 3000, 128, [3000, 0, 1, 511, 512, 513, 2999, 0]),
    (16, 8, 8, 4000, 64, "rand"),
]


@pytest.mark.parametrize("case", FP8, ids=lambda c: "B%d_Hq%d_Hkv%d_Skv%d_d%d" % c[:5])
def test_length_split_fp8_matches_oracle(api, dev, case):
    import torch
    B, Hq, Hkv, Skv, d, spec = case
    lengths = lengths_of(spec, B, Skv, 2 * B + Skv)
    data = si.make_decode_fp8(600 + B + Skv, B, Hq, Hkv, Skv, d)
    scale = si.default_scale(d)
    q = to_dev(data["q"], dev)
    k = torch.from_numpy(data["k"]).to(dev)
    v = torch.from_numpy(data["v"]).to(dev)
    ws = torch.full((api.attn_decode_varlen_workspace_bytes(B, Hq, Hkv, Skv, d),), 0x7F,
                    dtype=torch.uint8, device=dev)
    print("length-split fp8 decode", case[:5], flush=True)
    o, lse = api.attn_decode_fp8(q, k, v, data["k_scale"], data["v_scale"],
                                 seqlens_k=torch.from_numpy(lengths).to(dev), scale=scale,
                                 workspace=ws)
    torch.cuda.synchronize()
    assert header(ws, B) == expected_header(lengths, Skv, Hq, Hkv)
    o_ref, lse_ref = ref.decode_fp8(si.bf16_to_f64(data["q"]), data["k"], data["v"], scale,
                                    data["k_scale"], data["v_scale"], seqlens=lengths)
    assert_close(bf16_to_np(o), o_ref, f32_to_np(lse), lse_ref, str(case[:5]))


def test_length_split_skewed_workload_sampled(api, dev):
    """The skewed decode the benchmark times (B64 Hq32 Hkv8, capacity 32768,
    d128; one sequence of 32768 keys among 63 of 256), in the same launch
    configuration: the oracle checks the long sequence and four short ones.
    The cache is drawn on the GPU (seeded) and the checked rows copied back."""
    import torch
    B, Hq, Hkv, cap, d = 64, 32, 8, 32768, 128
    lens = [256] * 17 + [cap] + [256] * 46
    gen = torch.Generator(device=dev)
    gen.manual_seed(6)
    k, v = (torch.randn((B, cap, Hkv, d), generator=gen, device=dev, dtype=torch.float32)
            .to(torch.bfloat16) for _ in range(2))
    q = torch.randn((B, Hq, d), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
    seq = torch.tensor(lens, dtype=torch.int32, device=dev)
    scale = si.default_scale(d)
    print("skewed decode workload", flush=True)
    o, lse = api.attn_decode_varlen(q, k, v, seq, scale=scale)
    torch.cuda.synchronize()
    bits = lambda t: t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    o_np, lse_np = bf16_to_np(o), f32_to_np(lse)
    for b in (17, 0, 1, 40, 63):
        n = lens[b]
        data = dict(q=bits(q[b:b + 1]), k=bits(k[b:b + 1, :n]), v=bits(v[b:b + 1, :n]))
        o_ref, lse_ref = decode_varlen_ref(data, [n], scale)
        assert_close(o_np[b:b + 1], o_ref, lse_np[b:b + 1], lse_ref, "skewed workload b=%d" % b)
    assert np.all(np.isfinite(o_np)) and np.all(np.isfinite(lse_np))
    del k, v
    torch.cuda.empty_cache()
