"""Measurement of the scaled fp8 matrix instruction's accumulation (the reason the quantised
forward forms Q K^T on the bf16 instruction over the E4M3 values and uses the fp8 one only for
P.V). E4M3 operands whose products span many binades are multiplied on both instructions and
compared with the exact float64 product; the bf16 instruction (exact operands, fp32
accumulation) must be exact to fp32 rounding, the fp8 one is reported. Also the bf16
matrix-instruction throughput diagnostic that the bench's roofline is measured against."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from oracle import fp8 as ofp8                  # noqa: E402  (E4M3 code table only)


@pytest.fixture(scope="module")
def sla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_linear_hybrid_amd as s
    return s


def codes(rng, shape, spread):
    """Random E4M3 codes (no NaN): exponent fields within `spread` binades of the top."""
    e = rng.integers(max(1, 15 - spread), 16, size=shape)
    m = rng.integers(0, 8, size=shape)
    m = np.where((e == 15) & (m == 7), 6, m)
    s = rng.integers(0, 2, size=shape)
    return ((s << 7) | (e << 3) | m).astype(np.uint8)


@pytest.mark.parametrize("spread", [1, 4, 14])
def test_fp8_instruction_accumulation(sla, spread):
    rng = np.random.default_rng(spread)
    a = codes(rng, (32, 64), spread)
    b = codes(rng, (64, 32), spread)
    av, bv = ofp8.e4m3_decode(a), ofp8.e4m3_decode(b)
    exact = av @ bv
    scale = np.abs(av) @ np.abs(bv)                  # sum of |products| per entry
    c8, c16 = sla.sla_diag_fp8_mfma(torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda())
    torch.cuda.synchronize()
    e8 = np.abs(c8.cpu().numpy() - exact) / scale
    e16 = np.abs(c16.cpu().numpy() - exact) / scale
    print(f"exponent spread {spread} binades: fp8 instruction max error {e8.max():.2e} of "
          f"sum|products| (mean {e8.mean():.2e}); bf16 instruction {e16.max():.2e}", flush=True)
    assert np.isfinite(c8.cpu().numpy()).all()
    assert e16.max() <= 2e-7                        # fp32 accumulation of exact products


def test_mfma_rate_diagnostic(sla):
    """The matrix-instruction throughput loop runs and reports a rate between a tenth of and the
    published dense bf16 peak (2.5 PFLOP/s at 2.4 GHz)."""
    tf = sla.sla_diag_mfma_rate("cuda", blocks=512, iters=1024)
    print(f"bf16 32x32x16 matrix-instruction rate: {tf:.0f} TFLOP/s", flush=True)
    assert 250.0 < tf <= 2500.0 * 1.02
