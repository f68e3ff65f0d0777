"""attn_decode_noalloc (split partials in the library's fixed device scratch,
no allocation) against attn_decode with a caller workspace: the same kernels
and split count, so the same bits; and both within the parity bars of the fp64
oracle.  Two calls in a row, the second smaller, so what the first left in
the shared scratch cannot leak into the second's result."""
import numpy as np
import pytest

import synth_inputs as si
from oracle import cpu
from tests.gpu_util import assert_close, bf16_to_np, f32_to_np, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def api():
    from tiled_attention_transformer_amd import api as a
    a._lib.load()
    return a


CALLS = [  # B, Hq, Hkv, Skv, d, splits: the GQA decode workload's sizes in 8 chunks, then smaller
    (64, 32, 8, 4096, 128, 8),
    (3, 16, 4, 1000, 64, 7),
]


def _run(api, dev, case, seed):
    import torch
    B, Hq, Hkv, Skv, d, splits = case
    data = si.make_decode(seed, B, Hq, Hkv, Skv, d)
    q, k, v = (to_dev(data[x], dev) for x in "qkv")
    scale = si.default_scale(d)
    print("no-alloc decode", case, flush=True)
    o1 = torch.full_like(q, float("nan"))
    l1 = torch.full((B, Hq), float("nan"), dtype=torch.float32, device=dev)
    api.attn_decode_noalloc(q, k, v, o=o1, lse=l1, scale=scale, num_splits=splits)
    o2, l2 = api.attn_decode(q, k, v, scale=scale, num_splits=splits)
    torch.cuda.synchronize()
    assert api.attn_decode_workspace_bytes(B, Hq, Hkv, Skv, d, splits) > 0
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)
    o_ref, lse_ref = cpu.decode_full(data["q"], data["k"], data["v"], scale)
    assert_close(bf16_to_np(o1), o_ref, f32_to_np(l1), lse_ref, "no-alloc %s" % (case,))


def test_noalloc_decode_two_calls_second_smaller(api, dev):
    for i, case in enumerate(CALLS):
        _run(api, dev, case, seed=300 + i)


def test_noalloc_decode_library_choice_uses_no_scratch(api, dev):
    """The library's split choice at the workload's sizes is one chunk: the
    entry point then needs no scratch and matches attn_decode bit for bit."""
    import torch
    B, Hq, Hkv, Skv, d = 64, 32, 8, 4096, 128
    assert api.attn_decode_workspace_bytes(B, Hq, Hkv, Skv, d, 0) == 0
    data = si.make_decode(310, B, Hq, Hkv, Skv, d)
    q, k, v = (to_dev(data[x], dev) for x in "qkv")
    o1, l1 = api.attn_decode_noalloc(q, k, v, num_splits=0)
    o2, l2 = api.attn_decode(q, k, v, num_splits=0)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)
