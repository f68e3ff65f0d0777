"""GPU parity of attn_fwd_exp2_poly: part of each tile's exponentials by the
library's exp2 polynomial, against the fp64 oracle at the same bar as
attn_fwd (O within 2e-2 max-abs, LSE within 1e-3).  The polynomial's own
accuracy is pinned on the host (tests/test_exp2_poly.py)."""
import numpy as np
import pytest

import synth_inputs as si
from oracle import cpu
from tests.gpu_util import assert_close, bf16_to_np, f32_to_np, to_dev

pytestmark = pytest.mark.gpu

SHARES = [4, 8, 16]

CASES = [  # B, Sq, Skv, Hq, Hkv, d, causal
    (1, 300, 300, 2, 1, 128, True),       # ragged last query and key tiles, few items
    (2, 129, 257, 4, 2, 64, True),        # Sq < Skv, bottom-right causal, d = 64
    (1, 200, 77, 2, 2, 128, True),        # Sq > Skv: leading rows have no key
    (1, 1, 1, 1, 1, 64, True),            # smallest case
    (3, 65, 200, 6, 3, 128, False),
    (16, 300, 300, 16, 16, 128, True),    # more items than compute units
    (8, 260, 333, 32, 8, 128, False),
]


@pytest.fixture(scope="module")
def api():
    from tiled_attention_transformer_amd import api as a
    a._lib.load()
    return a


def run(api, dev, data, scale, causal, poly):
    import torch
    q, k, v = (to_dev(data[n], dev) for n in "qkv")
    B, Sq, Hq, _ = q.shape
    o = torch.full(q.shape, float("nan"), dtype=torch.bfloat16, device=dev)
    lse = torch.full((B, Hq, Sq), float("nan"), dtype=torch.float32, device=dev)
    if poly is None:
        api.attn_fwd(q, k, v, o=o, lse=lse, scale=scale, causal=causal)
    else:
        api.attn_fwd_exp2_poly(q, k, v, poly, o=o, lse=lse, scale=scale, causal=causal)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("poly", SHARES)
@pytest.mark.parametrize("case", CASES, ids=lambda c: "B%d_Sq%d_Skv%d_Hq%d_Hkv%d_d%d_%s" % (
    *c[:6], "causal" if c[6] else "full"))
def test_poly_share_matches_oracle(api, dev, case, poly):
    B, Sq, Skv, Hq, Hkv, d, causal = case
    data = si.make_prefill(500 + Sq + Skv, B, Hq, Hkv, Sq, Skv, d)
    scale = si.default_scale(d)
    o, lse = run(api, dev, data, scale, causal, poly)
    o, lse = bf16_to_np(o), f32_to_np(lse)
    o_ref, lse_ref = cpu.attn_full(data["q"], data["k"], data["v"], scale, causal)
    assert_close(o, o_ref, lse, lse_ref, "%s poly %d" % (case, poly))
    if causal and Sq > Skv:
        # rows with no key: the clamp makes every masked weight exactly 0
        assert np.all(o[:, :Sq - Skv] == 0)


def test_poly_zero_is_attn_fwd_bitwise(api, dev):
    import torch
    for case in ((16, 300, 300, 16, 16, 128, True), (1, 200, 77, 2, 2, 64, False)):
        B, Sq, Skv, Hq, Hkv, d, causal = case
        data = si.make_prefill(77, B, Hq, Hkv, Sq, Skv, d)
        o0, l0 = run(api, dev, data, 0.1, causal, 0)
        o1, l1 = run(api, dev, data, 0.1, causal, None)
        assert torch.equal(o0.view(torch.int16), o1.view(torch.int16)), case
        assert torch.equal(l0, l1), case


def test_poly_share_deterministic(api, dev):
    import torch
    data = si.make_prefill(78, 4, 8, 2, 513, 513, 128)
    a = run(api, dev, data, 0.09, True, 8)
    b = run(api, dev, data, 0.09, True, 8)
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16))
    assert torch.equal(a[1], b[1])


def test_poly_causal_prefill_workload_every_row(api, dev):
    """Workload 2 (B4 H16 S2048 d128, causal) with 4, 8 and 16 of each
    lane's 32 exponentials per tile on the polynomial: every row against the
    C oracle, and the distance to the hardware-exponential path printed for
    the record."""
    spec, data = si.make_workload("causal_prefill")
    o_ref, lse_ref = cpu.attn_full(data["q"], data["k"], data["v"], spec["scale"], True)
    o_hw, l_hw = run(api, dev, data, spec["scale"], True, None)
    o_hw, l_hw = bf16_to_np(o_hw), f32_to_np(l_hw)
    for poly in SHARES:
        o, lse = run(api, dev, data, spec["scale"], True, poly)
        o, lse = bf16_to_np(o), f32_to_np(lse)
        err = assert_close(o, o_ref, lse, lse_ref, "workload 2, poly %d" % poly)
        print("workload 2 poly %d: max|dO| %.4g max|dLSE| %.3g vs oracle; vs hardware exp2: "
              "max|dO| %.4g max|dLSE| %.3g" % (poly, *err, np.abs(o - o_hw).max(),
                                                 np.abs(lse - l_hw).max()), flush=True)


@pytest.mark.parametrize("spread", [2.0, 4.0, 8.0])
def test_poly_share_sharp_logits(api, dev, spread):
    """Logits at 2-8x the default spread (rows dominated by a few keys, most
    weights far below 1, where a polynomial's relative error matters most)
    with half of the exponentials on the polynomial: the same bars."""
    B, Sq, Skv, Hq, Hkv, d, causal = 2, 333, 333, 4, 2, 128, True
    scale = float(np.float32(spread / np.sqrt(d)))
    data = si.make_prefill(1500 + int(spread), B, Hq, Hkv, Sq, Skv, d)
    o, lse = run(api, dev, data, scale, causal, 16)
    o_ref, lse_ref = cpu.attn_full(data["q"], data["k"], data["v"], scale, causal)
    err = assert_close(bf16_to_np(o), o_ref, f32_to_np(lse), lse_ref, "sharp x%g poly 16" % spread)
    print("sharp logits x%g, poly 16 of 32: max|dO| %.4g max|dLSE| %.3g" % (spread, *err), flush=True)
