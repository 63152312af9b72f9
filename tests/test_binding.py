"""Argument checks of the Python binding that run before anything reaches the library: host
tensors are refused (a kernel would otherwise be handed host pointers)."""
import pytest

torch = pytest.importorskip("torch")

import sparse_linear_hybrid_amd as sla      # noqa: E402


def cpu_inputs(d=64):
    q = torch.zeros(1, 2, 128, d, dtype=torch.bfloat16)
    k = torch.zeros(1, 2, 256, d, dtype=torch.bfloat16)
    p = torch.zeros(d, d, dtype=torch.float32)
    a = torch.zeros(2, d, dtype=torch.float32)
    return q, k, k.clone(), p, p.clone(), a


@pytest.mark.parametrize("entry", ["sla_forward", "sla_forward_fp8", "sla_forward_pisa",
                                   "sla_forward_taylor", "sla_route", "sla_route_taylor"])
def test_host_tensors_are_refused(entry):
    q, k, v, pq, pk, al = cpu_inputs()
    f = getattr(sla, entry)
    args = {"sla_forward": (q, k, v, pq, pk, al, 2), "sla_forward_fp8": (q, k, v, pq, pk, al, 2),
            "sla_forward_pisa": (q, k, v, pq, pk, 2), "sla_forward_taylor": (q, k, v, al, 2),
            "sla_route": (q, k, pq, pk, 2), "sla_route_taylor": (q, k, 2)}[entry]
    with pytest.raises(ValueError, match="GPU tensor"):
        f(*args)
