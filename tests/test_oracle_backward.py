"""Pins of the backward oracle (gradients of the SLA2 forward at a fixed selection).

* central finite differences of the forward oracle's pieces, along random directions in
  Q, K, V and alpha (inputs kept away from the ReLU kink);
* top-k = every block and alpha = 1: the gradients of dense softmax attention, by torch
  autograd in float64 on the CPU (a library routine);
* top-k = 0 and alpha = 0: the gradients of plain ReLU linear attention written as one torch
  expression and differentiated by autograd;
* alpha's gradient alone, and the head-level wrapper against the head function.
"""
import math

import numpy as np
import pytest

from oracle import backward as bw
from oracle import sla_oracle as so

torch = pytest.importorskip("torch")
RNG = np.random.default_rng(2024)


def away_from_kink(x, gap=1e-2):
    """Move entries within `gap` of zero away from it (finite differences across the ReLU
    kink would not measure the one-sided derivative)."""
    x = x.copy()
    small = np.abs(x) < gap
    x[small] = np.where(x[small] >= 0, gap, -gap) * 5
    return x


def head(nq, nk, d, scale=1.0):
    q = away_from_kink(RNG.standard_normal((nq, d)) * scale)
    k = away_from_kink(RNG.standard_normal((nk, d)) * scale)
    v = RNG.standard_normal((nk, d))
    al = RNG.uniform(0.1, 0.9, d)
    return q, k, v, al


def random_selection(nbq, nbk, top_k):
    return np.stack([np.sort(RNG.choice(nbk, size=top_k, replace=False)) for _ in range(nbq)]) \
        .astype(np.int32).reshape(nbq, top_k)


@pytest.mark.parametrize("nq,nk,d,b,top_k", [(70, 150, 8, 32, 2), (64, 64 * 3 + 10, 16, 64, 1),
                                             (90, 100, 8, 32, 4)])
def test_gradients_match_central_differences(nq, nk, d, b, top_k):
    q, k, v, al = head(nq, nk, d)
    nbq, nbk = so.n_blocks(nq, b), so.n_blocks(nk, b)
    idx = random_selection(nbq, nbk, top_k)
    dout = RNG.standard_normal((nq, d))
    dq, dk, dv, dal = bw.backward_head(q, k, v, al, idx, b, dout)

    def loss(q_, k_, v_, al_):
        return float((dout * bw.forward_at(q_, k_, v_, al_, idx, b)[0]).sum())

    eps = 1e-6
    for name, grad in (("q", dq), ("k", dk), ("v", dv), ("alpha", dal)):
        for _ in range(3):
            args = {"q": q, "k": k, "v": v, "alpha": al}
            delta = RNG.standard_normal(args[name].shape)
            plus = dict(args, **{name: args[name] + eps * delta})
            minus = dict(args, **{name: args[name] - eps * delta})
            fd = (loss(plus["q"], plus["k"], plus["v"], plus["alpha"])
                  - loss(minus["q"], minus["k"], minus["v"], minus["alpha"])) / (2 * eps)
            an = float((grad * delta).sum())
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)


def test_all_blocks_alpha1_gives_dense_attention_gradients():
    nq, nk, d, b = 100, 150, 16, 32
    q, k, v, _ = head(nq, nk, d)
    al = np.ones(d)
    nbq, nbk = so.n_blocks(nq, b), so.n_blocks(nk, b)
    idx = np.tile(np.arange(nbk, dtype=np.int32), (nbq, 1))
    dout = RNG.standard_normal((nq, d))
    dq, dk, dv, _ = bw.backward_head(q, k, v, al, idx, b, dout)
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq[None, None], tk[None, None],
                                                         tv[None, None])[0, 0]
    (o * torch.tensor(dout)).sum().backward()
    for got, want in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        assert np.allclose(got, want.numpy(), rtol=1e-10, atol=1e-12)


def test_topk0_alpha0_gives_linear_attention_gradients():
    nq, nk, d, b = 80, 130, 8, 32
    q, k, v, _ = head(nq, nk, d)
    al = np.zeros(d)
    idx = np.zeros((so.n_blocks(nq, b), 0), np.int32)
    dout = RNG.standard_normal((nq, d))
    dq, dk, dv, dal = bw.backward_head(q, k, v, al, idx, b, dout)
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    fq, fk = torch.relu(tq), torch.relu(tk)
    o = (fq @ (fk.T @ tv)) / (fq @ fk.sum(0) + so.EPS)[:, None]
    (o * torch.tensor(dout)).sum().backward()
    for got, want in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        assert np.allclose(got, want.numpy(), rtol=1e-9, atol=1e-12)
    # with top-k = 0 the sparse output is zero, so dalpha = -sum dO (.) O_l
    assert np.allclose(dal, -(dout * o.detach().numpy()).sum(0), rtol=1e-10, atol=1e-12)


def test_alpha_gradient_is_the_branch_difference():
    nq, nk, d, b = 64, 200, 8, 32
    q, k, v, al = head(nq, nk, d)
    idx = random_selection(2, so.n_blocks(nk, b), 3)
    dout = RNG.standard_normal((nq, d))
    _, o_s, o_l = bw.forward_at(q, k, v, al, idx, b)
    dal = bw.backward_head(q, k, v, al, idx, b, dout)[3]
    assert np.allclose(dal, (dout * (o_s - o_l)).sum(0), rtol=1e-12, atol=1e-12)


def test_forward_at_matches_forward_oracle():
    from workloads import make_custom
    x = make_custom(1, 2, 100, 130, 8, 2, dtype="f32", block=32, seed=5)
    out, idx = so.forward(x)
    for h in range(2):
        o, _, _ = bw.forward_at(x.as_f64("q")[0, h], x.as_f64("k")[0, h], x.as_f64("v")[0, h],
                                x.alpha[h].astype(float), idx[0, h], 32)
        assert np.allclose(o, out[0, h], rtol=1e-13, atol=1e-15)


def test_backward_wrapper_matches_head_function():
    from workloads import make_custom
    x = make_custom(2, 2, 100, 130, 8, 2, dtype="f32", block=32, seed=6)
    dout = RNG.standard_normal((2, 2, 100, 8))
    dq, dk, dv, dal = bw.backward(x, dout)
    _, idx = so.forward(x)
    want_dal = np.zeros((2, 8))
    for b in range(2):
        for h in range(2):
            g = bw.backward_head(x.as_f64("q")[b, h], x.as_f64("k")[b, h], x.as_f64("v")[b, h],
                                 x.alpha[h].astype(float), idx[b, h], 32, dout[b, h])
            assert np.array_equal(dq[b, h], g[0]) and np.array_equal(dk[b, h], g[1])
            assert np.array_equal(dv[b, h], g[2])
            want_dal[h] += g[3]
    assert np.allclose(dal, want_dal, rtol=1e-14, atol=0)


def test_dq_blocks_equal_the_full_backward_rows():
    """The per-block dQ used for sampled checks at full size is the full backward's."""
    nq, nk, d, b = 200, 330, 16, 64
    q, k, v, al = head(nq, nk, d)
    idx = random_selection(so.n_blocks(nq, b), so.n_blocks(nk, b), 2)
    dout = RNG.standard_normal((nq, d))
    dq = bw.backward_head(q, k, v, al, idx, b, dout)[0]
    got = bw.dq_blocks(q, k, v, al, idx, b, dout, [0, 3])
    assert np.array_equal(got[0], dq[0:64]) and np.array_equal(got[3], dq[192:200])
