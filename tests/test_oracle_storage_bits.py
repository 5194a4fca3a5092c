"""Exact-bits pins of every storage point of the oracle's bf16 layer.

A tiny layer (3 tokens, d = 4, 2 experts of f = 4, top-2) is computed a
second time in exact rational arithmetic (fractions.Fraction) with this
file's own round-to-nearest-even to bf16, applied exactly where the layer
stores a value (reading r12/r12b):

    A  = rd(gelu(h))          G   = rd(gelu'(h))        Yp = rd(A W2)
    y  = rd(sum_j g_j Yp_j)   dYp = rd(g dy)            dA = dYp W2^T
    dH = rd(dA G)             dXp = rd(dH W1^T)         dx = rd(sum_j dXp_j)
    dW2 = rd(sum_a A_a^T dYp_a)                         dW1 = rd(sum_a x_a^T dH_a)

The inputs make every pre-activation h either 0, at least 12 or at most -40,
where gelu and gelu' are exact in fp64 (gelu(h) = h, gelu'(h) = 1 for
h >= 12; gelu(0) = 0, gelu'(0) = 1/2; both 0 for h <= -40), so the whole
chain is rational and the expected bits are unique.  Each storage point's
rounding is checked to change at least one value, so a dropped or moved
rounding fails.  A second test pins A and G at generic h against gelu and
gelu' written with math.erf."""
import math
from fractions import Fraction as Fr

import numpy as np

from block_sparse_gemm_amd import synth


def rd_bf16(q: Fr) -> Fr:
    """Round a rational to the nearest bf16 value, ties to even (normal
    range; the values here stay far from under- and overflow)."""
    if q == 0:
        return Fr(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fr(2) ** e > a:
        e -= 1
    # 8 significant bits: a = m * 2^(e - 7) with m in [128, 256)
    scale = Fr(2) ** (e - 7)
    m = a / scale
    lo = m.numerator // m.denominator
    rem = m - lo
    if rem > Fr(1, 2) or (rem == Fr(1, 2) and lo % 2 == 1):
        lo += 1
    return sign * lo * scale


def _bf16(rng, lo, hi, shape):
    v = rng.uniform(lo, hi, size=shape).astype(np.float32)
    return synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(v)).reshape(shape)


def _exact_case():
    T, d, E, f, k = 3, 4, 2, 4, 2
    rng = np.random.default_rng(2024)
    x = _bf16(rng, 1.0, 2.0, (T, d))
    # each hidden column: large positive (h >= 16), zero, or large negative
    # (h <= -48) for every token (x >= 1 > 0)
    W1 = np.zeros((d, E * f), np.float32)
    kinds = ["pos", "zero", "neg", "pos", "pos", "neg", "zero", "pos"]
    for c, kind in enumerate(kinds):
        if kind == "pos":
            W1[:, c] = _bf16(rng, 4.0, 8.0, (d,))
        elif kind == "neg":
            W1[:, c] = -_bf16(rng, 12.0, 16.0, (d,))
    W2 = _bf16(rng, -0.3, 0.3, (E * f, d))
    dy = _bf16(rng, -2.0, 2.0, (T, d))
    logits = np.array([[1.0, 0.5], [0.25, 2.0], [-1.0, 0.75]], np.float32)
    return T, d, E, f, k, x, W1, W2, dy, logits


def test_every_storage_point_bit_exact(orc):
    T, d, E, f, k, x, W1, W2, dy, logits = _exact_case()
    r = orc.route(logits, k, False)
    assert r["expert_idx"].tolist() == [0, 1, 1, 0, 1, 0]
    O = orc.make_layer(x, W1, W2, r, k, E, dy=dy, prec="bf16")
    assigns = np.arange(T * k)
    G_o, A_o, Yp_o = O.assign_forward(assigns)
    dYp_o, dH_o, dXp_o = O.assign_backward(assigns)
    y_o = O.forward_tokens(np.arange(T))
    dx_o = O.backward_tokens(np.arange(T))
    dW2_o = O.dW2_block(np.arange(E * f), np.arange(d))
    dW1_o = O.dW1_block(np.arange(d), np.arange(E * f))

    F = lambda v: Fr(float(v))
    changed = {}

    def store(name, exact):
        rounded = rd_bf16(exact)
        changed[name] = changed.get(name, False) or rounded != exact
        return rounded

    A, G, Yp, dYp, dH, dXp = {}, {}, {}, {}, {}, {}
    for a in range(T * k):
        t, e = a // k, int(r["expert_idx"][a])
        g = F(r["gate"][a])
        A[a], G[a], dH[a] = [], [], []
        for n in range(f):
            h = sum(F(x[t, i]) * F(W1[i, e * f + n]) for i in range(d))
            assert h == 0 or h >= 12 or h <= -40
            A[a].append(store("A", h if h > 0 else Fr(0)))
            G[a].append(store("G", Fr(1) if h > 0 else Fr(1, 2) if h == 0 else Fr(0)))
        Yp[a] = [store("Yp", sum(A[a][n] * F(W2[e * f + n, m]) for n in range(f)))
                 for m in range(d)]
        dYp[a] = [store("dYp", g * F(dy[t, m])) for m in range(d)]
        for n in range(f):
            dA = sum(dYp[a][m] * F(W2[e * f + n, m]) for m in range(d))
            dH[a].append(store("dH", dA * G[a][n]))
        dXp[a] = [store("dXp", sum(dH[a][n] * F(W1[i, e * f + n]) for n in range(f)))
                  for i in range(d)]
    y = [[store("y", sum(F(r["gate"][t * k + j]) * Yp[t * k + j][m] for j in range(k)))
          for m in range(d)] for t in range(T)]
    dx = [[store("dx", sum(dXp[t * k + j][i] for j in range(k))) for i in range(d)]
          for t in range(T)]
    dW2 = np.zeros((E * f, d), object)
    dW1 = np.zeros((d, E * f), object)
    for e in range(E):
        mine = [a for a in range(T * k) if r["expert_idx"][a] == e]
        for n in range(f):
            for m in range(d):
                dW2[e * f + n, m] = store("dW2", sum(A[a][n] * dYp[a][m] for a in mine))
            for i in range(d):
                dW1[i, e * f + n] = store("dW1", sum(F(x[a // k, i]) * dH[a][n] for a in mine))

    as_np = lambda rows: np.array([[float(v) for v in row] for row in rows])
    assert np.array_equal(A_o, as_np([A[a] for a in assigns]))
    assert np.array_equal(G_o, as_np([G[a] for a in assigns]))
    assert np.array_equal(Yp_o, as_np([Yp[a] for a in assigns]))
    assert np.array_equal(y_o, as_np(y))
    assert np.array_equal(dYp_o, as_np([dYp[a] for a in assigns]))
    assert np.array_equal(dH_o, as_np([dH[a] for a in assigns]))
    assert np.array_equal(dXp_o, as_np([dXp[a] for a in assigns]))
    assert np.array_equal(dx_o, as_np(dx))
    assert np.array_equal(dW2_o, dW2.astype(float))
    assert np.array_equal(dW1_o, dW1.astype(float))
    # every rounding point moves at least one value: dropping it would show
    for name in ("A", "Yp", "y", "dYp", "dH", "dXp", "dx", "dW2", "dW1"):
        assert changed[name], f"the {name} rounding changes nothing in this case"


def test_saved_activation_and_derivative_bits_at_generic_h(orc):
    """A = rd(gelu(h)) and G = rd(gelu'(h)) with h the exact pre-activation:
    gelu and gelu' evaluated here in fp64 with math.erf, rounded with this
    file's rounding; values within a few fp64 ulps of a bf16 rounding
    boundary (where the two fp64 evaluations may legitimately disagree) are
    skipped, and they must be rare."""
    T, d, E, f, k = 64, 8, 2, 32, 1
    rng = np.random.default_rng(7)
    x = _bf16(rng, -1.0, 1.0, (T, d))
    W1 = _bf16(rng, -0.8, 0.8, (d, E * f))
    W2 = _bf16(rng, -0.3, 0.3, (E * f, d))
    logits = rng.standard_normal((T, E)).astype(np.float32)
    r = orc.route(logits, k, False)
    O = orc.make_layer(x, W1, W2, r, k, E, dy=np.zeros((T, d), np.float32), prec="bf16")
    G_o, A_o, _ = O.assign_forward(np.arange(T * k))
    skipped = checked = 0
    for a in range(T * k):
        e = int(r["expert_idx"][a])
        for n in range(f):
            h = sum(Fr(float(x[a, i])) * Fr(float(W1[i, e * f + n])) for i in range(d))
            hf = float(h)
            cdf = 0.5 * (1.0 + math.erf(hf / math.sqrt(2.0)))
            pdf = math.exp(-0.5 * hf * hf) / math.sqrt(2.0 * math.pi)
            for got, val in ((A_o[a, n], hf * cdf), (G_o[a, n], cdf + hf * pdf)):
                want = rd_bf16(Fr(val))
                # the nearest rounding boundary lies half an ulp from the
                # result (ulp = 2^(e - 7) for |want| in [2^e, 2^(e+1)))
                ulp = 2.0 ** (math.frexp(float(want))[1] - 8) if want != 0 else 2.0 ** -133
                if abs(abs(Fr(val) - want) - Fr(ulp) / 2) <= abs(val) * 2.0 ** -48:
                    skipped += 1
                    continue
                checked += 1
                assert got == float(want), (a, n, hf, got, float(want))
    assert checked > 0.99 * (checked + skipped)
