"""The library's debug modes (environment variable ATTN_DEBUG, read at every
call), used to catch races in the prefill kernel's LDS ring:

* 2: every wave fills the ring stage its tile loads are about to land in
  with NaN first, so a read of a stage before its loads completed, or after
  the stage was handed back to the loads, shows up as NaN (here: as any
  change in the output);
* 4: the shallowest ring the pipeline allows (3 stages instead of 4), where
  every tile's loads must complete one phase after they start, so a missing
  or misplaced wait shows up at once;
* 6: both at once;
* 1: every call synchronises its stream and reports kernel faults as
  ATTN_ERR_HIP.

Modes 2 and 4 change nothing about the arithmetic: each must give the normal
mode's outputs bit for bit, on workloads with enough work items for the
ping-pong kernel (items >= compute units) and with ragged last tiles.  (At
d = 64 fixed batches run the single-group kernel, which has no debug
variants: there the check is that the flags change nothing.)
"""
import numpy as np
import pytest

import synth_inputs as si
from tests.gpu_util import bf16_to_np, f32_to_np, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def api():
    from tiled_attention_transformer_amd import api as a
    a._lib.load()
    return a


CASES = [  # B, S, Hq, Hkv, d, causal
    (4, 2048, 16, 16, 128, True),
    (3, 1500, 24, 24, 128, False),
    (2, 1300, 32, 8, 128, True),
    (4, 2048, 16, 16, 64, True),
    (3, 1111, 32, 4, 64, False),
]


def _run(api, q, k, v, causal):
    import torch
    o, lse = api.attn_fwd(q, k, v, scale=0.088, causal=causal)
    torch.cuda.synchronize()
    return bf16_to_np(o), f32_to_np(lse)


@pytest.mark.parametrize("mode", [2, 4, 6], ids=["poison", "ring3", "poison-ring3"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "B%dS%dH%d-%dd%d%s" % (
    *c[:5], "c" if c[5] else ""))
def test_debug_ring_modes_bitwise(api, dev, monkeypatch, case, mode):
    B, S, Hq, Hkv, d, causal = case
    data = si.make_prefill(41 + d, B, Hq, Hkv, S, S, d)
    q, k, v = (to_dev(data[x], dev) for x in "qkv")
    print("debug mode %d on %s" % (mode, case), flush=True)
    monkeypatch.delenv("ATTN_DEBUG", raising=False)
    o0, l0 = _run(api, q, k, v, causal)
    monkeypatch.setenv("ATTN_DEBUG", str(mode))
    o1, l1 = _run(api, q, k, v, causal)
    monkeypatch.delenv("ATTN_DEBUG")
    assert not np.isnan(o1).any() and not np.isnan(l1).any()
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)


def test_debug_sync_mode(api, dev, monkeypatch):
    """Mode 1: prefill (fixed and ragged) and decode return ATTN_OK after a
    stream synchronisation and give the same outputs."""
    import torch
    data = si.make_prefill(43, 2, 8, 8, 600, 600, 128)
    q, k, v = (to_dev(data[x], dev) for x in "qkv")
    monkeypatch.delenv("ATTN_DEBUG", raising=False)
    o0, l0 = _run(api, q, k, v, True)
    vl = si.make_varlen(44, 5, 1, 700, H=8, d=64)
    cu_d = torch.from_numpy(vl["cu_seqlens"]).to(dev)
    mx = int(np.diff(vl["cu_seqlens"]).max())
    vq, vk, vv = (to_dev(vl[x], dev) for x in "qkv")
    ov0, lv0 = api.attn_fwd_varlen(vq, vk, vv, cu_d, cu_d, mx, mx, scale=0.1, causal=True)
    dq = to_dev(np.ascontiguousarray(data["q"][:, 0]), dev)
    od0, ld0 = api.attn_decode(dq, k, v, scale=0.088)
    torch.cuda.synchronize()
    monkeypatch.setenv("ATTN_DEBUG", "1")
    o1, l1 = _run(api, q, k, v, True)
    ov1, lv1 = api.attn_fwd_varlen(vq, vk, vv, cu_d, cu_d, mx, mx, scale=0.1, causal=True)
    od1, ld1 = api.attn_decode(dq, k, v, scale=0.088)
    monkeypatch.delenv("ATTN_DEBUG")
    torch.cuda.synchronize()
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)
    assert torch.equal(ov0, ov1) and torch.equal(lv0, lv1)
    assert torch.equal(od0, od1) and torch.equal(ld0, ld1)
