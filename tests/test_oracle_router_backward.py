"""Pins of the oracle's gate backward (gradient of <dy, y> with respect to the
router logits, the top-k selection held fixed).

- torch fp64 autograd of softmax -> pick -> (renormalise) -> weighted sum;
- central finite differences of <dy, y> in the logits;
- properties that hold for any input: every row of dlogits sums to zero
  (softmax), and with renormalised gates the experts not picked get zero
  (the renormalised gates do not depend on them; up to fp64 rounding).
"""
import numpy as np
import pytest
import torch


def _case(orc, T=40, E=8, k=2, d=16, seed=0, renorm=False):
    rng = np.random.default_rng(seed)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    r = orc.route(logits, k, renorm)
    dy = rng.standard_normal((T, d)).astype(np.float32)
    yp = rng.standard_normal((T * k, d))
    return logits, r, dy, yp


def _autograd(logits, r, dy, yp, k, renorm):
    lg = torch.from_numpy(logits.astype(np.float64)).requires_grad_()
    T, E = lg.shape
    ei = torch.from_numpy(r["expert_idx"].astype(np.int64)).view(T, k)
    p = torch.softmax(lg, dim=1)
    g = torch.gather(p, 1, ei)
    if renorm:
        g = g / g.sum(dim=1, keepdim=True)
    y = (g[:, :, None] * torch.from_numpy(yp).view(T, k, -1)).sum(dim=1)
    (y * torch.from_numpy(dy.astype(np.float64))).sum().backward()
    return lg.grad.numpy()


@pytest.mark.parametrize("renorm", [False, True])
@pytest.mark.parametrize("k", [1, 2, 3])
def test_router_backward_equals_autograd(orc, renorm, k):
    logits, r, dy, yp = _case(orc, k=k, seed=k, renorm=renorm)
    got = orc.route_backward(logits, k, r["expert_idx"], dy, yp, renorm)
    want = _autograd(logits, r, dy, yp, k, renorm)
    assert np.max(np.abs(got - want)) <= 1e-12 * max(1.0, np.max(np.abs(want)))


@pytest.mark.parametrize("renorm", [False, True])
def test_router_backward_finite_differences(orc, renorm):
    logits, r, dy, yp = _case(orc, T=6, E=5, k=2, d=9, seed=7, renorm=renorm)
    T, E = logits.shape
    k = 2
    ei = r["expert_idx"].reshape(T, k)

    def loss(lg):
        # the same picks, gates recomputed from the perturbed logits (fp64)
        x = lg.astype(np.float64)
        p = np.exp(x - x.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        g = np.take_along_axis(p, ei, axis=1)
        if renorm:
            g = g / g.sum(axis=1, keepdims=True)
        y = (g[:, :, None] * yp.reshape(T, k, -1)).sum(axis=1)
        return float(np.sum(y * dy))

    got = orc.route_backward(logits, k, r["expert_idx"], dy, yp, renorm)
    h = 1e-3
    for t in range(T):
        for e in range(E):
            lp, lm = logits.astype(np.float64).copy(), logits.astype(np.float64).copy()
            lp[t, e] += h
            lm[t, e] -= h
            fd = (loss(lp) - loss(lm)) / (2 * h)
            assert abs(fd - got[t, e]) <= 1e-6 * max(1.0, abs(fd))


def test_router_backward_properties(orc):
    logits, r, dy, yp = _case(orc, T=64, E=16, k=2, d=32, seed=3)
    g = orc.route_backward(logits, 2, r["expert_idx"], dy, yp, False)
    assert np.max(np.abs(g.sum(axis=1))) <= 1e-12 * max(1.0, np.max(np.abs(g)))
    assert np.count_nonzero(g) == g.size  # every expert's logit moves its softmax
    logits, r, dy, yp = _case(orc, T=64, E=16, k=2, d=32, seed=3, renorm=True)
    g = orc.route_backward(logits, 2, r["expert_idx"], dy, yp, True)
    ei = r["expert_idx"].reshape(64, 2)
    picked = np.zeros_like(g, dtype=bool)
    np.put_along_axis(picked, ei, True, axis=1)
    # zero up to the rounding of the softmax term (exactly zero in exact arithmetic)
    assert np.max(np.abs(g[~picked])) <= 1e-14 * np.max(np.abs(g))
    assert np.max(np.abs(g.sum(axis=1))) <= 1e-12 * max(1.0, np.max(np.abs(g)))
