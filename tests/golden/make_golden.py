"""Write the stored oracle values under tests/golden/.

Calls only the oracle and the seeded input generator.  The pages print no
numeric worked example of attention, so these fixtures are oracle outputs
kept as a regression pin: a later change to the oracle's arithmetic that
moves them must say which passage justifies it.

Run from the repository root:  python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle import ref  # noqa: E402
import synth_inputs as si  # noqa: E402

CITATION = ('lecompute.fr, "FlashAttention-4 : limites du calcul matriciel", section '
            '"Entre deux multiplications il faut fabriquer les poids" (scores, softmax '
            'weights summing to one, second product mixing V); causal reach from section '
            '"Le FP4 ajoute un compromis numérique" read bottom-right.')

ROWS = [(0, 0, 0), (0, 0, 1), (0, 1, 127), (0, 1, 128), (0, 0, 255), (0, 1, 255)]


def tiny_case(causal):
    spec = dict(si.WORKLOADS["tiny"])
    data = si.make_prefill(spec["seed"], spec["B"], spec["Hq"], spec["Hkv"], spec["Sq"],
                           spec["Skv"], spec["d"])
    scale = si.default_scale(spec["d"])
    o, lse = ref.attention_rows(data["q"], data["k"], data["v"], scale, causal, ROWS)
    return dict(
        citation=CITATION,
        workload="B=1 Hq=Hkv=2 Sq=Skv=256 d=64, seed 1, bf16 N(0,1), scale=float32(1/8)",
        causal=causal, scale=scale, rows=ROWS,
        o=[[float(x) for x in r] for r in o], lse=[float(x) for x in lse])


def main():
    for causal in (False, True):
        name = "tiny_%s_rows.json" % ("causal" if causal else "noncausal")
        with open(os.path.join(HERE, name), "w") as f:
            json.dump(tiny_case(causal), f, indent=1)
        print("wrote", name)


if __name__ == "__main__":
    main()
