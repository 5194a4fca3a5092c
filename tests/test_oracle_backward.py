"""Pins of the oracle's backward pass (gradients of x, W1, W2 with the routing
and gates held fixed).

- torch fp64 autograd of the per-expert batched form (a library routine);
- central finite differences of <dy, y> (independent of any derivative code);
- experts that receive no token have exactly zero weight gradients;
- the bf16 storage points stay within a few bf16 ulps of the exact gradient.
"""
import numpy as np
import pytest
import torch

from block_sparse_gemm_amd import synth
from tests.test_oracle_float import small_layer


def autograd_grads(inp, r, k, E):
    x = torch.from_numpy(inp["x"]).double().requires_grad_()
    W1 = torch.from_numpy(inp["W1"]).double().requires_grad_()
    W2 = torch.from_numpy(inp["W2"]).double().requires_grad_()
    dy = torch.from_numpy(inp["dy"]).double()
    T, d = x.shape
    f = W1.shape[1] // E
    ei = torch.from_numpy(r["expert_idx"].astype(np.int64))
    g = torch.from_numpy(r["gate"].astype(np.float64))
    y = torch.zeros(T, d, dtype=torch.float64)
    for e in range(E):
        a = torch.nonzero(ei == e).flatten()
        if len(a) == 0:
            continue
        h = x[a // k] @ W1[:, e * f:(e + 1) * f]
        yp = torch.nn.functional.gelu(h) @ W2[e * f:(e + 1) * f]
        y = y.index_add(0, a // k, g[a, None] * yp)
    (y * dy).sum().backward()
    return x.grad.numpy(), W1.grad.numpy(), W2.grad.numpy()


def test_backward_equals_autograd_f64(orc):
    L, r, inp = small_layer(orc, T=120, d=128, E=4, f=256, k=2, seed=11)
    gx, gW1, gW2 = autograd_grads(inp, r, L.k, L.E)
    dx = L.backward_tokens(np.arange(L.T))
    assert np.max(np.abs(dx - gx)) <= 1e-12 * max(1, np.max(np.abs(gx)))
    rows = np.arange(0, L.E * L.f, 37)
    cols = np.arange(0, L.d, 13)
    dW2 = L.dW2_block(rows, cols)
    assert np.max(np.abs(dW2 - gW2[np.ix_(rows, cols)])) <= 1e-12 * max(1, np.max(np.abs(gW2)))
    rows1 = np.arange(0, L.d, 11)
    cols1 = np.arange(0, L.E * L.f, 29)
    dW1 = L.dW1_block(rows1, cols1)
    assert np.max(np.abs(dW1 - gW1[np.ix_(rows1, cols1)])) <= 1e-12 * max(1, np.max(np.abs(gW1)))


def test_backward_finite_differences(orc):
    L, r, inp = small_layer(orc, T=20, d=128, E=3, f=128, k=2, seed=12)
    dy = inp["dy"].astype(np.float64)
    base = dict(inp)

    def loss(**over):
        arrs = dict(base, **over)
        L2 = orc.make_layer(arrs["x"], arrs["W1"], arrs["W2"], r, L.k, L.E, dy=inp["dy"],
                            prec="f64")
        return float(np.sum(L2.forward_tokens(np.arange(L.T)) * dy))

    rng = np.random.default_rng(0)
    h = 1e-3  # fp32 inputs: perturb by an exactly representable step
    dx = L.backward_tokens(np.arange(L.T))
    for _ in range(4):
        t, i = rng.integers(L.T), rng.integers(L.d)
        xp, xm = inp["x"].copy(), inp["x"].copy()
        xp[t, i] += np.float32(h)
        xm[t, i] -= np.float32(h)
        step = float(xp[t, i]) - float(xm[t, i])
        fd = (loss(x=xp) - loss(x=xm)) / step
        assert abs(fd - dx[t, i]) <= 1e-5 * max(1, abs(fd))
    for _ in range(4):
        n, m = rng.integers(L.E * L.f), rng.integers(L.d)
        wp, wm = inp["W2"].copy(), inp["W2"].copy()
        wp[n, m] += np.float32(h)
        wm[n, m] -= np.float32(h)
        step = float(wp[n, m]) - float(wm[n, m])
        fd = (loss(W2=wp) - loss(W2=wm)) / step
        assert abs(fd - L.dW2_block([n], [m])[0, 0]) <= 1e-5 * max(1, abs(fd))
    for _ in range(4):
        i, c = rng.integers(L.d), rng.integers(L.E * L.f)
        wp, wm = inp["W1"].copy(), inp["W1"].copy()
        wp[i, c] += np.float32(h)
        wm[i, c] -= np.float32(h)
        step = float(wp[i, c]) - float(wm[i, c])
        fd = (loss(W1=wp) - loss(W1=wm)) / step
        assert abs(fd - L.dW1_block([i], [c])[0, 0]) <= 1e-5 * max(1, abs(fd))


def test_zero_token_expert_has_zero_weight_grads(orc):
    rng = np.random.default_rng(5)
    T, d, E, f, k = 40, 128, 4, 128, 1
    logits = rng.standard_normal((T, E)).astype(np.float32)
    logits[:, 2] = -100.0  # expert 2 never wins
    x = rng.standard_normal((T, d)).astype(np.float32)
    W1 = (rng.standard_normal((d, E * f)) * 0.05).astype(np.float32)
    W2 = (rng.standard_normal((E * f, d)) * 0.05).astype(np.float32)
    dy = rng.standard_normal((T, d)).astype(np.float32)
    r = orc.route(logits, k)
    assert r["counts"][2] == 0
    L = orc.make_layer(x, W1, W2, r, k, E, dy=dy)
    rows = np.arange(2 * f, 3 * f, 7)
    assert np.all(L.dW2_block(rows, np.arange(0, d, 5)) == 0)
    assert np.all(L.dW1_block(np.arange(0, d, 5), rows) == 0)
    assert np.any(L.dW2_block(np.arange(0, f, 7), [0, 1]) != 0)


def test_backward_bf16_close_to_exact(orc):
    L, r, inp = small_layer(orc, T=64, d=128, E=2, f=256, k=1, seed=13, prec="bf16")
    Lf = orc.make_layer(inp["x"], inp["W1"], inp["W2"], r, L.k, L.E, dy=inp["dy"], prec="f64")
    dx, dxf = L.backward_tokens(np.arange(64)), Lf.backward_tokens(np.arange(64))
    assert np.max(np.abs(dx - dxf)) <= 2e-2 * np.max(np.abs(dxf))
    rows, cols = np.arange(0, 512, 9), np.arange(0, 128, 7)
    a, b = L.dW2_block(rows, cols), Lf.dW2_block(rows, cols)
    assert np.max(np.abs(a - b)) <= 2e-2 * np.max(np.abs(b))
    rows1, cols1 = np.arange(0, 128, 7), np.arange(0, 512, 9)
    a, b = L.dW1_block(rows1, cols1), Lf.dW1_block(rows1, cols1)
    assert np.max(np.abs(a - b)) <= 2e-2 * np.max(np.abs(b))
    # per-assignment rows agree with the token-level dx (k = 1)
    dYp, dH, dXp = L.assign_backward(np.arange(64))
    assert np.array_equal(dXp, dx)
    q = lambda v: synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(v.astype(np.float32)))
    assert np.array_equal(dYp, q(r["gate"][:, None].astype(np.float64) * inp["dy"]))
