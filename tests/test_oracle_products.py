"""Pins of the oracle's block products (orc_sdd, orc_dsd, orc_dstd): on the
same stored inputs they must reproduce, value for value, the per-token layer
oracle (a different computation: one token's dense MLP at a time), whose own
pins are the library GEMMs, autograd and finite differences of the other
test files.  Both sum in fp64 in ascending order and round once at the same
storage point, so the comparisons are exact."""
import numpy as np
import pytest

from block_sparse_gemm_amd import synth

pytestmark = []


def _layer(orc, cfg, seed, empty=None):
    inp = synth.make_inputs(cfg, seed)
    if empty is not None:
        inp["logits"][:, empty] = -50.0
    r = orc.route(inp["logits"], cfg.k, cfg.renorm, cfg.bin_rows)
    O = orc.make_layer(inp["x"].values, inp["W1"].values, inp["W2"].values, r, cfg.k, cfg.E,
                       act=cfg.act, W3=inp["W3"].values if "W3" in inp else None,
                       dy=inp["dy"].values, prec=cfg.dtype, prec_yp=cfg.yp)
    return inp, r, O


def _rows(blocks, F, rows):
    """Full rows [len(rows), F*128] of a block-major array (block height
    from the array's shape)."""
    br = blocks.shape[1]
    b = blocks.reshape(-1, br, 128)
    base = (rows // br) * F
    return np.concatenate([b[base + j, rows % br] for j in range(F)], axis=1)


@pytest.mark.parametrize("br", [128, 64])
@pytest.mark.parametrize("act", ["gelu", "swiglu"])
def test_products_reproduce_the_per_token_oracle(orc, act, br):
    """Blocks of 128 rows over bins of 128, and blocks of 64 rows over bins
    of 64 (the block-size study)."""
    kw = dict(renorm=True) if act == "swiglu" else {}
    cfg = synth.LayerConfig("prod_pin", T=300, d=128, E=4, f=256, k=2, act=act, backward=True,
                            bin_rows=br, **kw)
    inp, r, O = _layer(orc, cfg, 3, empty=2)       # expert 2 gets no token
    E, F, d, f = cfg.E, cfg.f // 128, cfg.d, cfg.f
    bo = r["bin_offsets"]
    assert np.all(bo % br == 0)
    P = dict(block_rows=br)
    Tp = int(bo[E])
    assert r["counts"][2] == 0
    xp = orc.permute_pad(inp["x"].values, cfg.k, r["dest_row"], Tp, prec="bf16")
    dyp = orc.permute_pad(inp["dy"].values, cfg.k, r["dest_row"], Tp, scale=r["gate"],
                          prec="bf16")
    assigns = np.arange(cfg.T * cfg.k)
    rows = r["dest_row"][assigns].astype(np.int64)
    S, A_tok, Yp_tok = O.assign_forward(assigns)
    dYp_tok, dH_tok, dXp_tok = O.assign_backward(assigns)

    # first layer + activation (and the saved factors)
    if act == "gelu":
        A, G = orc.sdd(xp, inp["W1"].values, d, bo, E, F, "gelu", want_aux=True, **P)
        assert np.array_equal(_rows(G, F, rows), S)
    else:
        A, SQ = orc.sdd(xp, inp["W1"].values, d, bo, E, F, "silu_mul", b2=inp["W3"].values,
                        want_aux=True, **P)
        nnz = A.shape[0]
        assert np.array_equal(_rows(SQ[:nnz], F, rows), S[0])
        assert np.array_equal(_rows(SQ[nnz:], F, rows), S[1])
        G = SQ
    assert np.array_equal(_rows(A, F, rows), A_tok)
    # pad rows of A are gelu(0) = 0 / silu(0) * 0 = 0
    pad = np.nonzero(r["row_src"] < 0)[0]
    assert not np.any(_rows(A, F, pad))

    # second layer
    Yp = orc.dsd(A, bo, E, F, inp["W2"].values, d, **P)
    assert np.array_equal(Yp[rows], Yp_tok)
    assert np.array_equal(dyp[rows], dYp_tok)

    # backward first product: dA = dYp W2^T, times the saved factor(s)
    if act == "gelu":
        dH = orc.sdd(dyp, inp["W2"].values, d, bo, E, F, "gelu_bwd", trans_b=True, aux_in=G,
                     **P)
        assert np.array_equal(_rows(dH, F, rows), dH_tok)
        dXp = orc.dsd(dH, bo, E, F, inp["W1"].values, d, trans_b=True, **P)
        assert np.array_equal(dXp[rows], dXp_tok)
    else:
        dH = orc.sdd(dyp, inp["W2"].values, d, bo, E, F, "silu_mul_bwd", trans_b=True,
                     aux_in=G, **P)
        nnz = dH.shape[0] // 2
        assert np.array_equal(_rows(dH[:nnz], F, rows), dH_tok[0])   # gate projection
        assert np.array_equal(_rows(dH[nnz:], F, rows), dH_tok[1])   # up projection
        dXp = orc.dsd(dH[:nnz], bo, E, F, inp["W1"].values, d, trans_b=True, blocks2=dH[nnz:],
                      b2=inp["W3"].values, **P)
        # the two projections' sums may interleave differently: equal up to
        # one rounding of nearly equal fp64 sums
        np.testing.assert_allclose(dXp[rows], dXp_tok, rtol=2 ** -7, atol=1e-12)

    # weight gradients through the transpose index; the empty expert's are zero
    dW2 = orc.dstd(A, bo, E, F, dyp, d, **P)
    all_rows, all_cols = np.arange(E * f), np.arange(d)
    assert np.array_equal(dW2, O.dW2_block(all_rows, all_cols))
    dW1t = orc.dstd(dH if act == "gelu" else dH[:dH.shape[0] // 2], bo, E, F, xp, d, **P)
    assert np.array_equal(dW1t.T, O.dW1_block(all_cols, all_rows))
    assert not np.any(dW2[2 * f:3 * f]) and not np.any(dW1t[2 * f:3 * f])


def test_products_match_a_blockwise_brute_force(orc):
    """Tiny operands: every block of each product against numpy's fp64
    product of the block's row and column slices, rounded by the oracle's
    scalar rounding."""
    rng = np.random.default_rng(4)
    E, F, K, N = 3, 2, 64, 128
    bo = np.array([0, 256, 256, 384], np.int32)            # expert 1 empty
    Tp = int(bo[-1])
    q = lambda a: synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(a.astype(np.float32)))
    a = q(rng.standard_normal((Tp, K)))
    b = q(rng.standard_normal((K, E * F * 128)) * 0.1)
    owner = np.repeat(np.arange(E), np.diff(bo) // 128)
    rdv = np.vectorize(lambda v: orc.rd(v, "bf16"))
    got = orc.sdd(a, b, K, bo, E, F, "none")
    for blk in range(got.shape[0]):
        rb, j = divmod(blk, F)
        c = owner[rb] * F + j
        want = a[128 * rb:128 * rb + 128].astype(np.float64) @ b[:, 128 * c:128 * c + 128]
        assert np.array_equal(got[blk], rdv(want))
    blocks = q(rng.standard_normal((Tp // 128 * F, 128, 128)))
    w = q(rng.standard_normal((E * F * 128, N)) * 0.1)
    c = orc.dsd(blocks, bo, E, F, w, N)
    for rb in range(Tp // 128):
        e = owner[rb]
        dense = np.concatenate([blocks[rb * F + j] for j in range(F)], axis=1).astype(np.float64)
        want = dense @ w[e * F * 128:(e + 1) * F * 128]
        assert np.array_equal(c[128 * rb:128 * rb + 128], rdv(want))
    dm = q(rng.standard_normal((Tp, N)))
    C = orc.dstd(blocks, bo, E, F, dm, N)
    for e in range(E):
        for j in range(F):
            want = np.zeros((128, N))
            for rb in np.nonzero(owner == e)[0]:
                want += blocks[rb * F + j].astype(np.float64).T @ dm[128 * rb:128 * rb + 128]
            col = e * F + j
            assert np.array_equal(C[128 * col:128 * col + 128], rdv(want))
