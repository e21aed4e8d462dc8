"""Write the oracle's outputs for the tiny reference workload to tiny_b1_v4096_r32.json.

Calls only ``oracle`` and the seeded input generator. The pages print no
worked numerical example, so this file is a regression record of the oracle
(it fixes what the oracle computes today), not an independent pin. The
workload: B=1, K=7, V=4096, r=32, f32 base ~N(0, 2^2), E and W bf16
~N(0, 0.05^2), T=1, Philox seed 1234, offset 0, data seed 1234 -- the tiny
case of the drafting-alone setup ("brb-nv/TensorRT-LLM pull 27", section
"2. One fused kernel per draft position").

Run from the repository root:  python tests/golden/make_golden.py
"""
import hashlib
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from ancestral_draft_token_amd import inputs  # noqa: E402

SAMPLE_V = [0, 1, 2, 3, 511, 1024, 2047, 3000, 4095]


def main():
    w = inputs.tiny()
    res = oracle.draft_block(w)
    out = {
        "workload": w.name,
        "source": "oracle/dspark_oracle.c via tests/golden/make_golden.py",
        "tokens": res.tokens.tolist(),
        "margin": [[float(x) for x in row] for row in res.margin],
        "logits_sha256": hashlib.sha256(res.logits.tobytes()).hexdigest(),
        "sample_v": SAMPLE_V,
        "logits_sample": res.logits[0][:, SAMPLE_V].astype(float).tolist(),
        "q_at_token": [float(res.q[0, k, res.tokens[0, k]]) for k in range(w.K)],
        "q_sample": res.q[0][:, SAMPLE_V].tolist(),
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_b1_v4096_r32.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print("wrote", path)


if __name__ == "__main__":
    main()
