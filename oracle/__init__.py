"""CPU float64 oracle for SLA2 sparse-linear attention.

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the cpu_baseline
leg of bench.py, never by the GPU library. It shares no code with the GPU path; both are
fed from the separate ``workloads`` input generators.

What pins each part to something other than itself (``-m "not gpu"`` tests):

* sla_oracle (router, sparse and linear branches, mix): top-k = all and alpha = 1 against
  torch's SDPA in float64; top-k = 0 and alpha = 0 against textbook linear attention; both
  branches against a token-by-token brute force; closed-form router scores, planted ties,
  the projection's orientation, pooling over valid tokens only, permutation invariance,
  the direct complement against total minus selected, the mix's endpoints and affinity
  (tests/test_oracle_pins.py); boundary gaps and near-tie flags on hand-built score rows and
  against a Python sort (tests/test_oracle_wrappers.py). tests/golden/tiny_oracle.json
  (written by tests/golden/make_golden.py from this oracle) only guards against change; it
  pins nothing by itself.
* fp8 (quantised sparse branch, both readings): the E4M3 table and rounding rule
  exhaustively, the block-scale closed form, equal-logit and two-key closed forms, the
  visit-order-free definition against the online form (tests/test_oracle_fp8.py); a
  token-loop brute force, and on E4M3-exact inputs the distance from the unquantised
  forward within the P-rounding bound (tests/test_oracle_wrappers.py).
* taylor_scores / route_head_taylor: zero variance, a two-value variance closed form, the
  token-level attention mass to fourth order, the reduction to the dot-product router
  (tests/test_oracle_taylor.py).
* pisa: every block routed and constant key blocks give dense attention, unit values give
  unit output, the first-order error falls as the square of the spread, the block
  statistics by hand (tests/test_oracle_pisa.py).
* backward: central finite differences of the forward oracle, torch autograd of dense
  attention and of plain linear attention, dalpha as the branch difference
  (tests/test_oracle_backward.py).

No function here is without such a pin. The SoftTop-k of the pages' training has no
formula on the pages and is not implemented (parity unpinned).
"""
from . import sla_oracle, fp8, pisa, backward
from .sla_oracle import forward, route, route_head, forward_head
from .fp8 import forward_fp8

__all__ = ["sla_oracle", "fp8", "pisa", "backward", "forward", "route", "route_head", "forward_head", "forward_fp8"]
