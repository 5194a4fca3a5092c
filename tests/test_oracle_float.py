"""Pins of the oracle's forward floats.

- activations: textbook normal-CDF values (GeLU = x * Phi(x)), odd-part
  identities, finite differences of the derivative;
- rounding: against an integer bit-trick bf16 conversion and exact cases;
- the layer: the per-expert batched-GEMM formulation (George Lin's Blog,
  MegaBlocks/FlexMoE post, section 1.2: Output_i = Input_i @ W_i) computed
  with numpy/torch matmul; the E=1, k=1 special case equals a dense MLP
  (torch's own GeLU/SiLU); invariants (token permutation, exact power-of-two
  scaling of W2, zero pad rows).
"""
import math
import os

import numpy as np
import pytest
import torch

from block_sparse_gemm_amd import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_gelu_table(orc):
    rows = [l.split() for l in open(os.path.join(GOLD, "normal_cdf.txt")) if l[0] != "#"]
    for xs, ps in rows:
        x, p = float(xs), float(ps)
        assert abs(orc.gelu(x) - x * p) <= 1e-15
        assert abs(orc.gelu(-x) - (-x) * (1 - p)) <= 1e-15
    assert orc.gelu(0.0) == 0.0


def test_gelu_identities_and_grad(orc):
    for x in np.linspace(-6, 6, 61):
        # Phi(x) + Phi(-x) = 1  =>  gelu(x) - gelu(-x) = x
        assert abs(orc.gelu(x) - orc.gelu(-x) - x) <= 1e-14
        h = 1e-6
        fd = (orc.gelu(x + h) - orc.gelu(x - h)) / (2 * h)
        assert abs(orc.gelu_grad(x) - fd) <= 1e-8
    assert orc.gelu_grad(0.0) == 0.5


def test_silu(orc):
    for z in np.linspace(-8, 8, 33):
        # sigmoid(z) + sigmoid(-z) = 1  =>  silu(z) - silu(-z) = z
        assert abs(orc.silu(z) - orc.silu(-z) - z) <= 1e-13
    assert abs(orc.silu(math.log(3.0)) - 0.75 * math.log(3.0)) <= 1e-15
    assert orc.silu(0.0) == 0.0


def test_rounding(orc):
    rng = np.random.default_rng(0)
    v = (rng.standard_normal(20000) * np.exp(rng.uniform(-30, 30, 20000))).astype(np.float32)
    want = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(v))
    got = np.array([orc.rd(float(a), "bf16") for a in v], np.float32)
    assert np.array_equal(got, want)
    # ties go to even; exact values stay
    assert orc.rd(1.0 + 2 ** -8, "bf16") == 1.0
    assert orc.rd(1.0 + 3 * 2 ** -8, "bf16") == 1.0 + 2 ** -6
    assert orc.rd(-(1.0 + 3 * 2 ** -8), "bf16") == -(1.0 + 2 ** -6)
    assert orc.rd(1.0 + 2 ** -8 + 2 ** -40, "bf16") == 1.0 + 2 ** -7
    assert orc.rd(0.1, "f32") == float(np.float32(0.1))
    assert orc.rd(0.1, "f64") == 0.1
    assert orc.rd(2.0 ** -130, "bf16") == 2.0 ** -130  # subnormal range, exact
    assert orc.rd(3 * 2.0 ** -135, "bf16") == 2.0 ** -133  # 0.75 quanta -> 1


def small_layer(orc, T=300, d=128, E=4, f=256, k=2, act="gelu", prec="f64", seed=0,
                x_std=1.0, renorm=False):
    rng = np.random.default_rng(seed)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    x = rng.standard_normal((T, d)).astype(np.float32) * np.float32(x_std)
    W1 = (rng.standard_normal((d, E * f)) * 0.05).astype(np.float32)
    W3 = (rng.standard_normal((d, E * f)) * 0.05).astype(np.float32) if act == "swiglu" else None
    W2 = (rng.standard_normal((E * f, d)) * 0.05).astype(np.float32)
    dy = rng.standard_normal((T, d)).astype(np.float32)
    if prec == "bf16":
        q = lambda a: None if a is None else synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(a))
        x, W1, W3, W2, dy = q(x), q(W1), q(W3), q(W2), q(dy)
    r = orc.route(logits, k, renorm)
    L = orc.make_layer(x, W1, W2, r, k, E, act=act, W3=W3, dy=dy, prec=prec)
    return L, r, dict(logits=logits, x=x, W1=W1, W2=W2, W3=W3, dy=dy)


def batched_gemm_forward(x, W1, W2, W3, ei, gate, k, E, act, rnd=None):
    """Per-expert batched GEMM: gather each expert's tokens, two matmuls."""
    T, d = x.shape
    f = W1.shape[1] // E
    rnd = rnd or (lambda a: a)
    y = np.zeros((T, d))
    yp_all = np.zeros((T * k, d))
    for e in range(E):
        a = np.nonzero(ei == e)[0]
        if len(a) == 0:
            continue
        X = x[a // k].astype(np.float64)
        Hm = X @ W1[:, e * f:(e + 1) * f].astype(np.float64)
        if act == "gelu":
            Am = rnd(torch.nn.functional.gelu(torch.from_numpy(Hm)).numpy())
        else:
            U = X @ W3[:, e * f:(e + 1) * f].astype(np.float64)
            Am = rnd(torch.nn.functional.silu(torch.from_numpy(Hm)).numpy() * U)
        yp_all[a] = rnd(Am @ W2[e * f:(e + 1) * f].astype(np.float64))
    for a in range(T * k):
        y[a // k] += float(gate[a]) * yp_all[a]
    return rnd(y), yp_all


@pytest.mark.parametrize("act", ["gelu", "swiglu"])
def test_forward_equals_batched_gemm_f64(orc, act):
    L, r, inp = small_layer(orc, act=act)
    tokens = np.arange(L.T)
    y = L.forward_tokens(tokens)
    want, yp = batched_gemm_forward(inp["x"], inp["W1"], inp["W2"], inp["W3"], r["expert_idx"],
                                    r["gate"], L.k, L.E, act)
    assert np.max(np.abs(y - want)) <= 1e-12 * max(1.0, np.max(np.abs(want)))
    G, A, Yp = L.assign_forward(np.arange(L.T * L.k))
    assert np.max(np.abs(Yp - yp)) <= 1e-12 * max(1.0, np.max(np.abs(yp)))


def test_forward_bf16_within_one_ulp_of_batched_gemm(orc):
    L, r, inp = small_layer(orc, prec="bf16", seed=4)
    q = lambda a: synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(a.astype(np.float32))).astype(
        np.float64)
    want, yp = batched_gemm_forward(inp["x"], inp["W1"], inp["W2"], None, r["expert_idx"],
                                    r["gate"], L.k, L.E, "gelu", rnd=q)
    G, A, Yp = L.assign_forward(np.arange(L.T * L.k))
    # summation order differs (BLAS vs ascending), so a rounding may flip by
    # one bf16 ulp (2^-7 relative at most); nothing more
    assert np.all(np.abs(Yp - yp) <= np.abs(yp) * 2.0 ** -7 + 1e-30)
    assert np.mean(Yp == yp) > 0.95
    y = L.forward_tokens(np.arange(L.T))
    assert np.all(np.abs(y - want) <= 2 * np.abs(want) * 2.0 ** -7 + 1e-30)
    assert np.mean(y == want) > 0.9


@pytest.mark.parametrize("act", ["gelu", "swiglu"])
def test_single_expert_is_dense_mlp(orc, act):
    L, r, inp = small_layer(orc, T=64, E=1, k=1, act=act, seed=2)
    assert np.all(r["gate"] == 1.0)
    x = torch.from_numpy(inp["x"]).double()
    h = x @ torch.from_numpy(inp["W1"]).double()
    if act == "gelu":
        a = torch.nn.functional.gelu(h)
    else:
        a = torch.nn.functional.silu(h) * (x @ torch.from_numpy(inp["W3"]).double())
    want = (a @ torch.from_numpy(inp["W2"]).double()).numpy()
    y = L.forward_tokens(np.arange(64))
    assert np.max(np.abs(y - want)) <= 1e-12


def test_forward_invariants(orc):
    L, r, inp = small_layer(orc, T=120, prec="bf16", seed=9)
    y = L.forward_tokens(np.arange(120))
    # permuting the tokens (and their logits) permutes the outputs
    perm = np.random.default_rng(1).permutation(120)
    r2 = orc.route(inp["logits"][perm], L.k)
    L2 = orc.make_layer(inp["x"][perm], inp["W1"], inp["W2"], r2, L.k, L.E, dy=inp["dy"][perm])
    assert np.array_equal(L2.forward_tokens(np.arange(120)), y[perm])
    # scaling W2 by 2 scales every output by exactly 2 (roundings commute)
    L3 = orc.make_layer(inp["x"], inp["W1"], inp["W2"] * 2, r, L.k, L.E)
    assert np.array_equal(L3.forward_tokens(np.arange(120)), 2 * y)
    # a zero input row gives a zero output row (gelu(0) = 0: pad rows vanish)
    x0 = inp["x"].copy()
    x0[5] = 0
    L4 = orc.make_layer(x0, inp["W1"], inp["W2"], r, L.k, L.E)
    assert np.all(L4.forward_tokens([5]) == 0)


def test_forward_tokens_consistent_with_assignment_rows(orc):
    L, r, inp = small_layer(orc, T=50, prec="bf16", seed=5)
    G, A, Yp = L.assign_forward(np.arange(100))
    y = L.forward_tokens(np.arange(50))
    g = r["gate"].astype(np.float64)
    s = g[0::2, None] * Yp[0::2] + g[1::2, None] * Yp[1::2]
    q = lambda a: synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(a.astype(np.float32)))
    assert np.max(np.abs(y - s)) <= np.max(np.abs(s)) * 2.0 ** -7
    # stored A and G are the activation and its derivative at h = x W1 (a
    # numpy product here), each to one bf16 rounding; the derivative from
    # torch autograd of the exact GeLU
    a = np.arange(100)
    e = r["expert_idx"][a]
    W1 = inp["W1"].astype(np.float64).reshape(L.d, L.E, L.f)
    h = np.einsum("ai,aif->af", inp["x"].astype(np.float64)[a // 2], W1[:, e, :].transpose(1, 0, 2))
    ht = torch.from_numpy(h).requires_grad_()
    gl = torch.nn.functional.gelu(ht)
    gl.sum().backward()
    assert np.max(np.abs(A - q(gl.detach().numpy()))) <= np.max(np.abs(A)) * 2.0 ** -7
    assert np.max(np.abs(G - q(ht.grad.numpy()))) <= np.max(np.abs(G)) * 2.0 ** -7
