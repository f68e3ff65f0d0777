"""The entry points under HIP graph capture.

A caller may capture the library's launches in a graph (the reason the
no-allocation decode exists).  The calls below are captured once, on a side
stream, with every buffer allocated beforehand; the graph is then replayed
several times, with the caller's own eager work, output poisoning and
synchronisations between replays, and every replay must give the bits of the
eager calls: a causal prefill, the same with a polynomial share of the
exponentials, the no-allocation decode (its fixed scratch,
an explicit 8-way split with the merge kernel), a decode with the caller's
workspace, and a decode split by the per-sequence lengths (whose kernel
rewrites the workspace header every call).  Nothing in the library records a
memory fill into a graph.
"""
import numpy as np
import pytest

import synth_inputs as si
from tests.gpu_util import to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def api():
    from tiled_attention_transformer_amd import api as a
    a._lib.load()
    return a


def test_graph_replays_match_eager(api, dev):
    import torch
    scale = si.default_scale(128)
    pre = si.make_prefill(5, 2, 8, 2, 300, 300, 128)
    q, k, v = (to_dev(pre[x], dev) for x in "qkv")
    dec = si.make_decode(6, 8, 16, 4, 2000, 128)
    dq, dk, dv = (to_dev(dec[x], dev) for x in "qkv")
    ragged = si.make_decode(7, 16, 8, 2, 4096, 128)
    rq, rk, rv = (to_dev(ragged[x], dev) for x in "qkv")
    lengths = torch.tensor([4096, 3, 0, 700, 2048, 1, 4000, 512] * 2, dtype=torch.int32, device=dev)

    # outputs and workspaces, allocated before any capture
    o_p, l_p = torch.empty_like(q), torch.empty((2, 8, 300), dtype=torch.float32, device=dev)
    o_e, l_e = torch.empty_like(q), torch.empty((2, 8, 300), dtype=torch.float32, device=dev)
    o_n, l_n = torch.empty_like(dq), torch.empty((8, 16), dtype=torch.float32, device=dev)
    o_w, l_w = torch.empty_like(dq), torch.empty((8, 16), dtype=torch.float32, device=dev)
    ws_w = torch.empty(api.attn_decode_workspace_bytes(8, 16, 4, 2000, 128, 8), dtype=torch.uint8,
                       device=dev)
    o_r, l_r = torch.empty_like(rq), torch.empty((16, 8), dtype=torch.float32, device=dev)
    ws_r = torch.empty(api.attn_decode_varlen_workspace_bytes(16, 8, 2, 4096, 128), dtype=torch.uint8,
                       device=dev)

    def calls(stream=None):
        api.attn_fwd(q, k, v, o=o_p, lse=l_p, scale=scale, causal=True, stream=stream)
        api.attn_fwd_exp2_poly(q, k, v, 8, o=o_e, lse=l_e, scale=scale, causal=True, stream=stream)
        api.attn_decode_noalloc(dq, dk, dv, o=o_n, lse=l_n, scale=scale, num_splits=8, stream=stream)
        api.attn_decode(dq, dk, dv, o=o_w, lse=l_w, scale=scale, num_splits=8, workspace=ws_w,
                        stream=stream)
        api.attn_decode_varlen(rq, rk, rv, lengths, o=o_r, lse=l_r, scale=scale, workspace=ws_r,
                               stream=stream)

    outs = (o_p, l_p, o_e, l_e, o_n, l_n, o_w, l_w, o_r, l_r)
    calls()                          # eager (also looks up the no-allocation scratch)
    torch.cuda.synchronize()
    eager = [t.clone() for t in outs]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls(side)                  # warm-up on the capture stream
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        calls(side)
    torch.cuda.synchronize()

    for rep in range(4):
        # the caller's own eager work between replays: poison the outputs and
        # the workspaces, and run something else on the device
        for t in outs:
            t.view(torch.uint8).fill_(0x7F)
        ws_w.fill_(0x55)
        ws_r.fill_(0x55)
        x = torch.randn(256, 256, device=dev)
        (x @ x).sum().item()
        g.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(("prefill O", "prefill LSE", "poly-share O", "poly-share LSE",
                                    "no-alloc O", "no-alloc LSE",
                                    "decode O", "decode LSE", "by-length O", "by-length LSE"),
                                   outs, eager):
            assert torch.equal(got.view(torch.uint8), want.view(torch.uint8)), \
                "replay %d: %s differs from the eager call" % (rep, name)
    # the by-length decode's empty sequence stays O = 0, LSE = -inf
    assert np.all(np.isneginf(l_r[2].cpu().numpy())) and torch.count_nonzero(o_r[2]).item() == 0
