"""The oracle still reproduces its stored values (tests/golden/)."""
import json
import os

import numpy as np
import pytest

from oracle import cpu, ref
import synth_inputs as si

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


@pytest.mark.parametrize("name", ["tiny_noncausal_rows.json", "tiny_causal_rows.json"])
def test_oracle_reproduces_stored_rows(name):
    g = json.load(open(os.path.join(GOLDEN, name)))
    assert "FlashAttention-4" in g["citation"]
    spec = si.WORKLOADS["tiny"]
    data = si.make_prefill(spec["seed"], spec["B"], spec["Hq"], spec["Hkv"], spec["Sq"],
                           spec["Skv"], spec["d"])
    for fn in (ref.attention_rows, cpu.attn_rows):
        o, lse = fn(data["q"], data["k"], data["v"], g["scale"], g["causal"], g["rows"])
        np.testing.assert_allclose(o, np.array(g["o"]), atol=1e-12, rtol=0)
        np.testing.assert_allclose(lse, np.array(g["lse"]), atol=1e-12, rtol=0)
    if g["causal"]:      # row 0 of a causal head is v_0 exactly
        v = si.bf16_to_f64(data["v"])
        np.testing.assert_allclose(g["o"][0], v[0, 0, 0], atol=1e-15)
