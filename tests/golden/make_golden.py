"""Writes tests/golden/tiny_oracle.json: the oracle's result on the 'tiny' workload
(B=1, H=2, N=1024, d=64, fp32 inputs, block 64, top-k 4, seed 0).

Calls only the oracle and the input generators. The pages print no worked example, so this
fixture is a regression record of the pinned oracle, not an independent pin.
"""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle import forward, forward_fp8          # noqa: E402
from workloads import make_inputs, sha256_of    # noqa: E402

ROWS = [0, 1, 63, 64, 500, 1000, 1023]


def main():
    x = make_inputs("tiny")
    out, idx = forward(x)
    out8, _ = forward_fp8(x, rows=np.array(ROWS))
    rec = {
        "workload": "tiny", "seed": 0,
        "inputs_sha256": sha256_of(x.q, x.k, x.v, x.proj_q, x.proj_k, x.alpha),
        "idx": idx.tolist(),
        "rows": ROWS,
        "out_rows": [[repr(float(v)) for v in out[0, h, r]] for h in range(2) for r in ROWS],
        "out_fp8_rows": [[repr(float(v)) for v in out8[0, h, r]] for h in range(2) for r in ROWS],
        "rms": repr(float(np.sqrt(np.mean(out ** 2)))),
    }
    with open(os.path.join(HERE, "tiny_oracle.json"), "w") as f:
        json.dump(rec, f, indent=0)


if __name__ == "__main__":
    main()
