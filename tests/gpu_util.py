"""Helpers shared by the GPU tests: moving bf16 bit arrays to and from torch."""
import numpy as np

import synth_inputs as si

O_TOL = 2e-2      # max-abs error on bf16 O against the unrounded fp64 oracle
LSE_TOL = 1e-3    # max-abs error on fp32 LSE


def to_dev(bits: np.ndarray, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)


def bf16_to_np(t) -> np.ndarray:
    """bf16 torch tensor -> float64 numpy (exact)."""
    import torch
    bits = t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return si.bf16_to_f64(bits)


def f32_to_np(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def assert_close(o_gpu, o_ref, lse_gpu=None, lse_ref=None, what=""):
    """Max-abs check on O (and LSE, where both are finite; -inf must match)."""
    err_o = float(np.abs(o_gpu - o_ref).max()) if o_ref.size else 0.0
    assert np.all(np.isfinite(o_gpu)), what + ": non-finite O"
    assert err_o <= O_TOL, "%s: max |dO| = %.4g > %g" % (what, err_o, O_TOL)
    err_l = 0.0
    if lse_ref is not None:
        fin = np.isfinite(lse_ref)
        assert np.array_equal(fin, np.isfinite(lse_gpu)), what + ": LSE finiteness differs"
        assert np.all(np.isneginf(lse_gpu[~fin])), what + ": masked LSE must be -inf"
        if fin.any():
            err_l = float(np.abs(lse_gpu[fin] - lse_ref[fin]).max())
        assert err_l <= LSE_TOL, "%s: max |dLSE| = %.4g > %g" % (what, err_l, LSE_TOL)
    return err_o, err_l


def sample_rows(B, Hq, Sq, n, seed, extra_rows=()):
    """(b, h, i) triples: tile edges, first/last rows and n random ones."""
    rng = np.random.default_rng(seed)
    rows = set()
    for i in list(extra_rows) + [0, 1, Sq - 1, Sq - 2, min(127, Sq - 1), min(128, Sq - 1)]:
        if 0 <= i < Sq:
            rows.add((int(rng.integers(B)), int(rng.integers(Hq)), int(i)))
    for _ in range(n):
        rows.add((int(rng.integers(B)), int(rng.integers(Hq)), int(rng.integers(Sq))))
    return np.array(sorted(rows), dtype=np.int64)


def decode_varlen_ref(data, lengths, scale):
    """The oracle's decode of sequence b over its first lengths[b] keys
    (O = 0, LSE = -inf for an empty sequence)."""
    from oracle import cpu
    B, Hq, d = data["q"].shape
    o = np.zeros((B, Hq, d))
    lse = np.full((B, Hq), -np.inf)
    for b, L in enumerate(lengths):
        if L > 0:
            ob, lb = cpu.decode_full(data["q"][b:b + 1], data["k"][b:b + 1, :L],
                                     data["v"][b:b + 1, :L], scale)
            o[b], lse[b] = ob[0], lb[0]
    return o, lse
