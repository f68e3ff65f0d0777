"""The seeded input generator: bf16 rounding and reproducibility."""
import numpy as np
import torch

import synth_inputs as si


def test_bf16_rounding_matches_torch():
    """Round-to-nearest-even to bf16 agrees with torch's own float32->bfloat16 cast."""
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * s for s in (1e-3, 1, 1e3)])
    # values exactly halfway between two bf16 numbers exercise the tie rule
    hi = np.concatenate([np.arange(0x3F00, 0x4100), np.arange(0xBF00, 0xC100)]).astype(np.uint32)
    ties = ((hi << np.uint32(16)) | np.uint32(0x8000)).view(np.float32)
    x = np.concatenate([x, ties[np.isfinite(ties)]])
    ours = si.f32_to_bf16_bits(x)
    theirs = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)
    back = si.bf16_to_f32(ours)
    assert np.all(np.abs(back - x) <= np.abs(x) * 2.0 ** -8 + 1e-45)


def test_generators_are_reproducible_and_shaped():
    a = si.make_prefill(7, 2, 4, 2, 5, 9, 8)
    b = si.make_prefill(7, 2, 4, 2, 5, 9, 8)
    for n in "qkv":
        assert np.array_equal(a[n], b[n])
    assert a["q"].shape == (2, 5, 4, 8) and a["k"].shape == (2, 9, 2, 8)
    c = si.make_prefill(8, 2, 4, 2, 5, 9, 8)
    assert not np.array_equal(a["q"], c["q"])
    d = si.make_decode(4, 3, 4, 2, 10, 8)
    assert d["q"].shape == (3, 4, 8) and d["v"].shape == (3, 10, 2, 8)


def test_head_scaled_keys():
    a = si.make_prefill(3, 1, 4, 4, 6, 6, 8, k_head_scale=True)
    c = a["k_head_scale"]
    assert c.shape == (4,) and np.all((c >= 0.5) & (c < 2.0))
    rng = np.random.default_rng(3)
    rng.standard_normal((1, 6, 4, 8), dtype=np.float32)
    k = rng.standard_normal((1, 6, 4, 8), dtype=np.float32)
    assert np.array_equal(a["k"], si.f32_to_bf16_bits(k * c[None, None, :, None]))


def test_varlen_lengths_drawn_first_inclusive():
    spec = si.WORKLOADS["ragged"]
    rng = np.random.default_rng(spec["seed"])
    lengths = rng.integers(spec["lo"], spec["hi"] + 1, spec["nseq"])
    assert lengths.min() >= 128 and lengths.max() <= 8192 and len(lengths) == 16
    small = si.make_varlen(1, 4, 2, 6, H=2, d=4)
    assert small["cu_seqlens"][0] == 0 and np.all(np.diff(small["cu_seqlens"]) >= 2)
    assert small["q"].shape[0] == small["cu_seqlens"][-1]
    assert small["cu_seqlens"].dtype == np.int32


def test_fp8_cache_generator():
    a = si.make_decode_fp8(11, 2, 4, 2, 50, 16)
    b = si.make_decode_fp8(11, 2, 4, 2, 50, 16)
    for n in ("q", "k", "v"):
        assert np.array_equal(a[n], b[n])
    assert a["k"].dtype == np.uint8 and a["k"].shape == (2, 50, 2, 16)
    assert a["q"].dtype == np.uint16 and a["q"].shape == (2, 4, 16)
    for n in ("k", "v"):
        c = a[n]
        assert not np.any((c & 0x7F) == 0x7F), "no NaN codes"
        assert np.any((c & 0x7F) == 0x7E), "the largest magnitude (448) is used"
        assert a[n + "_scale"] > 0 and np.isfinite(a[n + "_scale"])
        # the scale is float32: max|x| / 448
        assert np.float32(a[n + "_scale"]) == a[n + "_scale"]


def test_kmeans_generator():
    a = si.make_kmeans(2, 100, 7, 16)
    b = si.make_kmeans(2, 100, 7, 16)
    assert np.array_equal(a["x"], b["x"]) and np.array_equal(a["c"], b["c"])
    assert a["x"].shape == (100, 16) and a["c"].shape == (7, 16) and a["x"].dtype == np.uint16
    assert a["label"].min() >= 0 and a["label"].max() < 7
