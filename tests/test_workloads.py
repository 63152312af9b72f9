"""Input generators: storage rounding, determinism, shapes and structure."""
import numpy as np
import pytest

from workloads import (CONFIGS, bf16_bits_to_f32, bf16_round_bits, make_custom, make_inputs,
                       sha256_of)


def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 1e3,
                        np.array([0.0, -0.0, 1.0, 65504.0, 1e-30, 3.0e38], np.float32)])
    ours = bf16_round_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(bf16_bits_to_f32(ours), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_bf16_rounding_exhaustive():
    """Every finite bf16 value converts back to itself; the exact midpoint between two
    neighbours rounds to the one with an even last bit, and one float32 ulp either side of it
    rounds to the nearer neighbour (round to nearest, ties to even)."""
    bits = np.arange(1 << 16, dtype=np.uint32)
    exp_all_ones = (bits & 0x7F80) == 0x7F80
    finite = bits[~exp_all_ones]
    f = (finite << 16).view(np.float32)
    assert np.array_equal(bf16_round_bits(f), finite.astype(np.uint16))
    # midpoints between finite neighbours of the same sign (the successor of the largest
    # finite value is infinity, which is not a neighbour here)
    lo = finite[((finite + 1) & 0x7F80) != 0x7F80]
    lo = lo[(lo & 0x7FFF) != 0x7FFF]
    mid = ((lo << 16) + 0x8000).view(np.float32)
    even = np.where(lo & 1, lo + 1, lo).astype(np.uint16)
    assert np.array_equal(bf16_round_bits(mid), even)
    below = ((lo << 16) + 0x7FFF).view(np.float32)
    above = ((lo << 16) + 0x8001).view(np.float32)
    assert np.array_equal(bf16_round_bits(below), lo.astype(np.uint16))
    assert np.array_equal(bf16_round_bits(above), (lo + 1).astype(np.uint16))


def test_tiny_is_deterministic_and_shaped():
    a = make_inputs("tiny")
    b = make_inputs("tiny")
    assert sha256_of(a.q, a.k, a.v, a.proj_q, a.proj_k, a.alpha) == sha256_of(b.q, b.k, b.v, b.proj_q, b.proj_k, b.alpha)
    assert a.q.shape == (1, 2, 1024, 64) and a.q.dtype == np.float32
    assert a.proj_q.shape == (64, 64) and a.alpha.shape == (2, 64)
    assert np.all((a.alpha > 0) & (a.alpha < 1))
    assert abs(a.q.std() - 1) < 0.02 and abs(a.proj_q.std() * 8 - 1) < 0.05


def test_head_truncation_keeps_heads():
    a = make_inputs("video95", heads=1)
    b = make_inputs("video95", heads=2)
    assert np.array_equal(a.q[0, 0], b.q[0, 0]) and np.array_equal(a.v[0, 0], b.v[0, 0])
    assert a.q.dtype == np.uint16 and a.q.shape == (1, 1, 32768, 128)
    q = bf16_bits_to_f32(a.q[0, 0]).astype(np.float64)
    # smooth field: neighbouring tokens along x are strongly correlated
    c = np.corrcoef(q[:-1, 0], q[1:, 0])[0, 1]
    assert c > 0.8


def test_problem_block_counts():
    assert CONFIGS["video90"].nbk == 1182 and CONFIGS["video90"].n_kv % 64 == 16
    assert CONFIGS["video95"].nbk == 512
    assert CONFIGS["longctx"].nbq == 1 and CONFIGS["longctx"].nbk == 2048
    assert abs(CONFIGS["video95"].sparsity - (1 - 26 / 512)) < 1e-12


def test_custom_shapes():
    x = make_custom(2, 3, 100, 200, 64, 2, dtype="bf16", kind="smooth")
    assert x.q.shape == (2, 3, 100, 64) and x.k.shape == (2, 3, 200, 64)
    assert x.q.dtype == np.uint16
