"""Pins of the oracle's SwiGLU backward (gradients of x, W1 (gate
projection), W3 (up projection) and W2, the routing and gates held fixed).

- silu': central finite differences of silu, torch autograd, and the identity
  silu'(z) + silu'(-z) = 1 (from silu(z) - silu(-z) = z);
- the layer: torch fp64 autograd of the per-expert form
  (silu(X W1_e) * (X W3_e)) W2_e combined with the gates, including the
  per-assignment pre-activation gradients of both projections;
- central finite differences of <dy, y> in x, W1 and W3;
- the saved factors silu(h) and u * silu'(h) against numpy products + torch;
- experts without tokens get exactly zero gradients; bf16 storage stays
  within a few bf16 ulps of the exact gradients.
"""
import numpy as np
import torch

from block_sparse_gemm_amd import synth
from tests.test_oracle_float import small_layer


def test_silu_grad(orc):
    z = torch.linspace(-9, 9, 73, dtype=torch.float64, requires_grad=True)
    torch.nn.functional.silu(z).sum().backward()
    for zi, gi in zip(z.detach().numpy(), z.grad.numpy()):
        assert abs(orc.silu_grad(zi) - gi) <= 1e-14
        h = 1e-6
        fd = (orc.silu(zi + h) - orc.silu(zi - h)) / (2 * h)
        assert abs(orc.silu_grad(zi) - fd) <= 1e-8
        assert abs(orc.silu_grad(zi) + orc.silu_grad(-zi) - 1.0) <= 1e-14
    assert orc.silu_grad(0.0) == 0.5


def autograd_swiglu(inp, r, k, E):
    """Gradients of <dy, y> through the per-expert form in torch fp64, plus
    the gradients of each assignment's two pre-activations."""
    t = lambda key: torch.from_numpy(inp[key]).double().requires_grad_()
    x, W1, W3, W2 = t("x"), t("W1"), t("W3"), t("W2")
    dy = torch.from_numpy(inp["dy"]).double()
    T, d = x.shape
    f = W1.shape[1] // E
    ei = torch.from_numpy(r["expert_idx"].astype(np.int64))
    g = torch.from_numpy(r["gate"].astype(np.float64))
    y = torch.zeros(T, d, dtype=torch.float64)
    pre = []
    for e in range(E):
        a = torch.nonzero(ei == e).flatten()
        if len(a) == 0:
            continue
        h = x[a // k] @ W1[:, e * f:(e + 1) * f]
        u = x[a // k] @ W3[:, e * f:(e + 1) * f]
        h.retain_grad()
        u.retain_grad()
        pre.append((a, h, u))
        yp = (torch.nn.functional.silu(h) * u) @ W2[e * f:(e + 1) * f]
        y = y.index_add(0, a // k, g[a, None] * yp)
    (y * dy).sum().backward()
    dh = np.zeros((2, T * k, f))
    for a, h, u in pre:
        dh[0, a.numpy()] = h.grad.numpy()
        dh[1, a.numpy()] = u.grad.numpy()
    return x.grad.numpy(), W1.grad.numpy(), W3.grad.numpy(), W2.grad.numpy(), dh


def _rel(a, b):
    return np.max(np.abs(a - b)) / max(1.0, np.max(np.abs(b)))


def test_swiglu_backward_equals_autograd_f64(orc):
    L, r, inp = small_layer(orc, T=96, d=128, E=3, f=256, k=2, act="swiglu", seed=21,
                            renorm=True)
    gx, gW1, gW3, gW2, gdh = autograd_swiglu(inp, r, L.k, L.E)
    assert _rel(L.backward_tokens(np.arange(L.T)), gx) <= 1e-12
    dYp, dH, dXp = L.assign_backward(np.arange(L.T * L.k))
    assert dH.shape == (2, L.T * L.k, L.f)
    assert _rel(dH[0], gdh[0]) <= 1e-12  # gate projection
    assert _rel(dH[1], gdh[1]) <= 1e-12  # up projection
    rows, cols = np.arange(0, L.E * L.f, 23), np.arange(0, L.d, 9)
    assert _rel(L.dW2_block(rows, cols), gW2[np.ix_(rows, cols)]) <= 1e-12
    assert _rel(L.dW1_block(cols, rows), gW1[np.ix_(cols, rows)]) <= 1e-12
    assert _rel(L.dW3_block(cols, rows), gW3[np.ix_(cols, rows)]) <= 1e-12


def test_swiglu_backward_finite_differences(orc):
    L, r, inp = small_layer(orc, T=16, d=128, E=2, f=128, k=2, act="swiglu", seed=22)
    dy = inp["dy"].astype(np.float64)

    def loss(**over):
        a = dict(inp, **over)
        L2 = orc.make_layer(a["x"], a["W1"], a["W2"], r, L.k, L.E, act="swiglu", W3=a["W3"],
                            dy=inp["dy"], prec="f64")
        return float(np.sum(L2.forward_tokens(np.arange(L.T)) * dy))

    def fd(key, idx):
        p, m = inp[key].copy(), inp[key].copy()
        p[idx] += np.float32(1e-3)
        m[idx] -= np.float32(1e-3)
        step = float(p[idx]) - float(m[idx])
        return (loss(**{key: p}) - loss(**{key: m})) / step

    rng = np.random.default_rng(1)
    dx = L.backward_tokens(np.arange(L.T))
    for _ in range(3):
        t, i = int(rng.integers(L.T)), int(rng.integers(L.d))
        want = fd("x", (t, i))
        assert abs(want - dx[t, i]) <= 1e-5 * max(1, abs(want))
    for key, grad in (("W1", L.dW1_block), ("W3", L.dW3_block)):
        for _ in range(3):
            i, c = int(rng.integers(L.d)), int(rng.integers(L.E * L.f))
            want = fd(key, (i, c))
            assert abs(want - grad([i], [c])[0, 0]) <= 1e-5 * max(1, abs(want)), key
    for _ in range(3):
        n, m = int(rng.integers(L.E * L.f)), int(rng.integers(L.d))
        want = fd("W2", (n, m))
        assert abs(want - L.dW2_block([n], [m])[0, 0]) <= 1e-5 * max(1, abs(want))


def test_swiglu_saved_factors(orc):
    L, r, inp = small_layer(orc, T=40, d=128, E=2, f=256, k=2, act="swiglu", prec="bf16",
                            seed=23)
    a = np.arange(80)
    G, A, _ = L.assign_forward(a)
    assert G.shape == (2, 80, L.f)
    e = r["expert_idx"][a]
    X = inp["x"].astype(np.float64)[a // 2]
    W1 = inp["W1"].astype(np.float64).reshape(L.d, L.E, L.f)
    W3 = inp["W3"].astype(np.float64).reshape(L.d, L.E, L.f)
    h = np.stack([X[q] @ W1[:, e[q], :] for q in range(80)])
    u = np.stack([X[q] @ W3[:, e[q], :] for q in range(80)])
    ht = torch.from_numpy(h).requires_grad_()
    s = torch.nn.functional.silu(ht)
    s.sum().backward()
    q = lambda v: synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(v.astype(np.float32)))
    s = s.detach().numpy()
    assert np.max(np.abs(G[0] - q(s))) <= np.max(np.abs(G[0])) * 2.0 ** -7
    assert np.max(np.abs(G[1] - q(u * ht.grad.numpy()))) <= np.max(np.abs(G[1])) * 2.0 ** -7
    assert np.max(np.abs(A - q(s * u))) <= np.max(np.abs(A)) * 2.0 ** -7


def test_swiglu_zero_token_expert(orc):
    rng = np.random.default_rng(6)
    T, d, E, f, k = 40, 128, 3, 128, 1
    logits = rng.standard_normal((T, E)).astype(np.float32)
    logits[:, 1] = -100.0
    w = lambda *s: (rng.standard_normal(s) * 0.05).astype(np.float32)
    x, W1, W3, W2 = rng.standard_normal((T, d)).astype(np.float32), w(d, E * f), w(d, E * f), \
        w(E * f, d)
    dy = rng.standard_normal((T, d)).astype(np.float32)
    r = orc.route(logits, k)
    assert r["counts"][1] == 0
    L = orc.make_layer(x, W1, W2, r, k, E, act="swiglu", W3=W3, dy=dy)
    cols = np.arange(f, 2 * f, 5)
    assert np.all(L.dW3_block(np.arange(0, d, 7), cols) == 0)
    assert np.all(L.dW1_block(np.arange(0, d, 7), cols) == 0)
    assert np.all(L.dW2_block(cols, np.arange(0, d, 7)) == 0)
    assert np.any(L.dW3_block(np.arange(0, d, 7), np.arange(0, f, 5)) != 0)


def test_swiglu_bf16_close_to_exact(orc):
    L, r, inp = small_layer(orc, T=64, d=128, E=2, f=256, k=1, act="swiglu", prec="bf16",
                            seed=24)
    Lf = orc.make_layer(inp["x"], inp["W1"], inp["W2"], r, 1, 2, act="swiglu", W3=inp["W3"],
                        dy=inp["dy"], prec="f64")
    toks = np.arange(64)
    dx, dxf = L.backward_tokens(toks), Lf.backward_tokens(toks)
    assert np.max(np.abs(dx - dxf)) <= 2e-2 * np.max(np.abs(dxf))
    rows, cols = np.arange(0, 128, 7), np.arange(0, 512, 9)
    for name in ("dW1_block", "dW3_block"):
        a, b = getattr(L, name)(rows, cols), getattr(Lf, name)(rows, cols)
        assert np.max(np.abs(a - b)) <= 2e-2 * np.max(np.abs(b)), name
    a, b = L.dW2_block(cols, rows), Lf.dW2_block(cols, rows)
    assert np.max(np.abs(a - b)) <= 2e-2 * np.max(np.abs(b))
    # k = 1: the per-assignment input gradient is the token's
    _, dH, dXp = L.assign_backward(toks)
    assert np.array_equal(dXp, dx)
    assert dH.shape == (2, 64, 256)
