"""Write tiny_f32_oracle.json: oracle outputs on the tiny fp32 workload.

Calls only the oracle and the seeded input generator.
    python tests/golden/make_golden.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from softmax_attention_ut_amd.inputs import CONFIGS, generate_config  # noqa: E402


def main():
    cfg = CONFIGS["tiny_f32"]
    inp = generate_config(cfg)
    out, lse, _, _ = oracle.recurrent(inp.q, inp.k, inp.v, inp.w, inp.beta, inp.log_f, cfg.scale)
    rec = {"workload": "tiny_f32 (B=1, H=1, L=64, d=16, seed 0, scale 1/4)",
           "source": "oracle.recurrent (fp64)",
           "out": [[round(float(x), 15) for x in row] for row in out[0, 0]],
           "lse": [round(float(x), 15) for x in lse[0, 0]]}
    with open(os.path.join(HERE, "tiny_f32_oracle.json"), "w") as f:
        json.dump(rec, f, indent=0)


if __name__ == "__main__":
    main()
