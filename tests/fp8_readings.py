"""How far the two readings of the quantised sparse branch move the output (CPU, oracle only).

    python tests/fp8_readings.py [--heads 0 5 11] [--blocks 2]

On sampled query blocks of the video95 inputs it evaluates the unquantised forward, the
power-of-two reading (E8M0 block scales, P per query row and key tile; the GPU path) and the
literal reading (float32 absmax/448 block scales, one absmax/448 P scale per 64 x 64 tile,
ascending online softmax), and prints max-abs / RMS and relative RMS distance between each
pair. Information for the choice of reading; no test depends on it.
"""
import argparse
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from oracle import fp8                      # noqa: E402
from oracle import sla_oracle as so         # noqa: E402
from workloads import make_inputs           # noqa: E402


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="video95")
    ap.add_argument("--heads", type=int, nargs="+", default=[0, 5, 11])
    ap.add_argument("--blocks", type=int, default=2)
    args = ap.parse_args()
    x = make_inputs(args.workload, heads=max(args.heads) + 1)
    p = x.problem
    rng = np.random.default_rng(3)
    res = {"exact": [], "pow2": [], "literal": []}
    for h in args.heads:
        blocks = rng.choice(p.nbq, size=args.blocks, replace=False)
        rows = np.concatenate([np.arange(i * 64, min(i * 64 + 64, p.n_q)) for i in blocks])
        res["exact"].append(so.forward(x, heads=[(0, h)], rows=rows)[0][0, h, rows])
        res["pow2"].append(fp8.forward_fp8(x, heads=[(0, h)], rows=rows)[0][0, h, rows])
        res["literal"].append(fp8.forward_fp8_literal(x, heads=[(0, h)], rows=rows)[0][0, h, rows])
    r = {k: np.concatenate(v) for k, v in res.items()}
    rms = float(np.sqrt(np.mean(r["exact"] ** 2)))
    print(f"{args.workload}: heads {args.heads}, {args.blocks} query blocks each "
          f"({r['exact'].shape[0]} rows), output RMS {rms:.4f}")
    print(f"{'pair':24s} {'max-abs/RMS':>12s} {'RMS-rel':>10s}")
    for a, b in (("pow2", "exact"), ("literal", "exact"), ("pow2", "literal")):
        d = r[a] - r[b]
        print(f"{a + ' vs ' + b:24s} {np.abs(d).max() / rms:12.3e} "
              f"{np.sqrt(np.mean(d ** 2)) / rms:10.3e}")


if __name__ == "__main__":
    main()
