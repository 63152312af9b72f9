"""The oracle still reproduces its recorded result on the tiny workload."""
import json
import os

import numpy as np

from oracle import forward, forward_fp8
from workloads import make_inputs, sha256_of

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_tiny_golden():
    rec = json.load(open(os.path.join(HERE, "tiny_oracle.json")))
    x = make_inputs("tiny")
    assert sha256_of(x.q, x.k, x.v, x.proj_q, x.proj_k, x.alpha) == rec["inputs_sha256"]
    out, idx = forward(x)
    assert np.array_equal(idx, np.array(rec["idx"], np.int32))
    rows = rec["rows"]
    want = np.array([[float(v) for v in r] for r in rec["out_rows"]])
    got = np.array([out[0, h, r] for h in range(2) for r in rows])
    assert np.allclose(got, want, rtol=1e-12, atol=1e-14)
    out8, _ = forward_fp8(x, rows=np.array(rows))
    want8 = np.array([[float(v) for v in r] for r in rec["out_fp8_rows"]])
    got8 = np.array([out8[0, h, r] for h in range(2) for r in rows])
    assert np.allclose(got8, want8, rtol=1e-12, atol=1e-14)
