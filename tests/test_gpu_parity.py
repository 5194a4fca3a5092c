"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bars: integer outputs (routing, bins, placement, row_src, topology, the
permuted copy Xp, the scaled copy dYp) bit-exact; bf16 floats within
|gpu - oracle| <= 1e-2 * max(1, |oracle|) elementwise (plus a reported
self-check max|d| / max|o|); fp32 floats within max|d| <= 1e-4 * max|o| per
tensor.  Small cases compare every element; the five full-size workloads
compare every integer output and sampled float outputs (sampled tokens,
assignments and weight-gradient entries, chosen to include the smallest
and largest experts and the first and last token).
"""
import dataclasses

import numpy as np
import pytest
import torch

from block_sparse_gemm_amd import synth

pytestmark = pytest.mark.gpu

BF16_TOL = 1e-2
F32_TOL = 1e-4


def _say(msg):
    print(msg, flush=True)


def check_float(name, got, want, dtype, report):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert got.shape == want.shape, (name, got.shape, want.shape)
    d = np.abs(got - want)
    scale = max(np.max(np.abs(want)), 1e-30) if want.size else 1.0
    rel = float(np.max(d) / scale) if want.size else 0.0
    report[name] = rel
    if dtype == "bf16":
        bad = d > BF16_TOL * np.maximum(1.0, np.abs(want))
        assert not bad.any(), f"{name}: {bad.sum()} elements out of tolerance, max|d|={d.max()}"
        assert rel <= 1e-2, f"{name}: self-check max|d|/max|o| = {rel}"
    else:
        assert np.max(d) <= F32_TOL * scale, f"{name}: max|d|={d.max()} vs {F32_TOL * scale}"


@dataclasses.dataclass
class Case:
    cfg: synth.LayerConfig
    logits: np.ndarray = None      # override of the drawn logits
    n_tokens: int = 0              # 0 = every token
    n_wgrad: int = 0               # 0 = every weight-gradient entry


def make_case_inputs(case: Case, seed=0):
    inp = synth.make_inputs(case.cfg, seed)
    if case.logits is not None:
        inp["logits"] = np.ascontiguousarray(case.logits, np.float32)
    return inp


def run_gpu(cfg, inp):
    from block_sparse_gemm_amd import layer
    s = layer.Shape.of(cfg)
    L = layer.Layer(s)
    up = lambda key: layer.from_numpy(inp[key], cfg.dtype) if key in inp else None
    x, W1, W2, W3, dy = up("x"), up("W1"), up("W2"), up("W3"), up("dy")
    logits = torch.from_numpy(inp["logits"]).cuda()
    L.forward(x, logits, W1, W2, W3)
    if cfg.backward:
        L.backward(dy, W1, W2, W3)
    torch.cuda.synchronize()
    return L, dict(x=x, W1=W1, W2=W2, W3=W3, dy=dy, logits=logits)


def sample_assignments(cfg, r, n_tokens, seed=1):
    if n_tokens == 0 or n_tokens >= cfg.T:
        toks = np.arange(cfg.T)
    else:
        toks = synth.sample_tokens(cfg.T, n_tokens, seed)
        # add a token of the smallest non-empty and of the largest expert
        ei = r["expert_idx"]
        counts = r["counts"]
        nz = np.nonzero(counts)[0]
        for e in (nz[np.argmin(counts[nz])], int(np.argmax(counts))):
            a = int(np.nonzero(ei == e)[0][-1])
            toks = np.union1d(toks, [a // cfg.k])
    assigns = (toks[:, None] * cfg.k + np.arange(cfg.k)[None, :]).reshape(-1)
    return toks.astype(np.int64), assigns.astype(np.int64)


def wgrad_samples(cfg, r, n, seed=2):
    rng = np.random.default_rng(seed)
    Ef = cfg.E * cfg.f
    if n == 0:
        return np.arange(Ef), np.arange(cfg.d)
    # rows of dW2 (columns of dW1): include the smallest, the largest and an
    # empty expert when there is one
    counts = r["counts"]
    ex = [int(np.argmin(counts)), int(np.argmax(counts))]
    rows = set(rng.choice(Ef, size=n, replace=False).tolist())
    for e in ex:
        rows.update([e * cfg.f, e * cfg.f + cfg.f - 1])
    cols = set(rng.choice(cfg.d, size=min(n, cfg.d), replace=False).tolist()) | {0, cfg.d - 1}
    return np.array(sorted(rows)), np.array(sorted(cols))


def check_case(orc, case: Case, seed=0):
    cfg = case.cfg
    _say(f"[parity] case {cfg.name} T={cfg.T} d={cfg.d} E={cfg.E} f={cfg.f} k={cfg.k} "
         f"act={cfg.act} dtype={cfg.dtype} bwd={cfg.backward} seed={seed}")
    inp = make_case_inputs(case, seed)
    L, dev = run_gpu(cfg, inp)
    from block_sparse_gemm_amd import layer
    f64 = layer.to_numpy_f64
    report = {}

    # ---- routing, bins, placement: bit-exact
    r = orc.route(inp["logits"], cfg.k, cfg.renorm, cfg.bin_rows)
    for key, t in (("expert_idx", L.expert_idx), ("dest_row", L.dest_row), ("counts", L.counts),
                   ("bin_offsets", L.bin_offsets)):
        assert np.array_equal(t.cpu().numpy(), r[key]), key
    g = L.gate.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(g - r["gate"]) <= 1e-5 * np.abs(r["gate"]) + 1e-12), "gate"
    Tp = int(r["bin_offsets"][cfg.E])
    assert np.array_equal(L.row_src[:Tp].cpu().numpy(), r["row_src"]), "row_src"

    # ---- topology: bit-exact (blocks of 64 rows go with bins of 64)
    F = cfg.f // 128
    BR = 64 if cfg.bin_rows == 64 else 128
    Q = 256 // BR
    t = orc.topology(r["bin_offsets"], cfg.E, F, BR)
    nnz, R = t["nnz"], Tp // BR
    meta = L.topo.meta.cpu().numpy()
    assert meta[0] == nnz and meta[1] == R
    assert np.array_equal(L.topo.row_ptr[:R + 1].cpu().numpy(), t["row_ptr"])
    assert np.all(L.topo.row_ptr[R + 1:].cpu().numpy() == nnz)
    for key in ("col_idx", "row_idx", "trans_idx"):
        assert np.array_equal(getattr(L.topo, key)[:nnz].cpu().numpy(), t[key]), key
    assert np.array_equal(L.topo.col_ptr.cpu().numpy(), t["col_ptr"]), "col_ptr"
    # the products' schedule: each expert's block rows Q at a time (256 rows),
    # the tiles in groups of G (from Tp_max and E), each entry with its place
    # in its group, the group's size and the tile's block rows
    rpe = L.Tp_max // (256 * cfg.E)
    G = 8 if (rpe >= 8 and cfg.E <= 16) else 4 if rpe >= 4 else 2 if rpe >= 2 else 1
    want_tiles = []
    for e in range(cfg.E):
        s0, s1 = r["bin_offsets"][e] // BR, r["bin_offsets"][e + 1] // BR
        starts = list(range(s0, s1, Q))
        for j, r0 in enumerate(starts):
            off = j % G
            size = min(G, len(starts) - (j - off))
            want_tiles.append((r0 << 8) | ((size - 1) << 5) | (off << 2) | (min(Q, s1 - r0) - 1))
    assert meta[3] == len(want_tiles)
    assert L.topo.row_tiles[:len(want_tiles)].cpu().numpy().tolist() == want_tiles
    # the weight-gradient schedule: experts by descending row blocks, ties to
    # the lower id
    rb = np.diff(r["bin_offsets"]) // BR
    want_order = sorted(range(cfg.E), key=lambda e: (-rb[e], e))
    assert L.topo.expert_order.cpu().numpy().tolist() == want_order, "expert_order"

    # ---- permuted, padded copy: bit-exact
    prec = cfg.dtype
    xp_want = orc.permute_pad(inp["x"].values, cfg.k, r["dest_row"], Tp, prec=prec)
    assert np.array_equal(f64(L.xp[:Tp]), xp_want), "xp"
    del xp_want

    # ---- forward floats
    toks, assigns = sample_assignments(cfg, r, case.n_tokens)
    O = orc.make_layer(inp["x"].values, inp["W1"].values, inp["W2"].values, r, cfg.k, cfg.E,
                       act=cfg.act, W3=inp["W3"].values if "W3" in inp else None,
                       dy=inp["dy"].values if "dy" in inp else None, prec=prec, prec_yp=cfg.yp)
    G, A, Yp = O.assign_forward(assigns)
    rows = torch.from_numpy(r["dest_row"][assigns]).cuda()
    check_float("A", f64(L.sparse_rows(L.act, rows)), A, prec, report)
    sw = cfg.act == "swiglu"
    if cfg.backward and sw:  # the saved factors silu(g), u * silu'(g)
        check_float("S", f64(L.sparse_rows(L.plane(L.gp, 0), rows)), G[0], prec, report)
        check_float("Q", f64(L.sparse_rows(L.plane(L.gp, 1), rows)), G[1], prec, report)
    elif cfg.backward:
        check_float("G", f64(L.sparse_rows(L.gp, rows)), G, prec, report)
    # the bar follows the workload's arithmetic (bf16 operands, fp32
    # accumulation) even where Yp is stored in fp32.  A forward-only top-1
    # layer writes y alone (its DSD's rows reach y through the combine, so
    # y carries them)
    yp_written = cfg.backward or not L.fuse_top1
    if yp_written:
        check_float("Yp", f64(L.yp[rows.long()]), Yp, prec, report)
    check_float("y", f64(L.y[torch.from_numpy(toks).cuda()]), O.forward_tokens(toks), prec,
                report)
    # pad rows of A and Yp are exactly zero
    pad = torch.from_numpy(np.nonzero(r["row_src"] < 0)[0]).cuda()
    if len(pad):
        if yp_written:
            assert torch.count_nonzero(L.yp[pad.long()]).item() == 0, "Yp pad rows"
        assert torch.count_nonzero(L.sparse_rows(L.act, pad)).item() == 0, "A pad rows"

    # ---- backward floats
    if cfg.backward:
        dYp, dH, dXp = O.assign_backward(assigns)
        # dYp = rd(gate * dy) uses each side's own gate (compared with a
        # tolerance above), so it is a float comparison here; the scaled copy
        # itself is checked bit-exact with a shared scale in
        # test_permute_pad_scaled_exact
        check_float("dYp", f64(L.dyp[rows.long()]), dYp, prec, report)
        if sw:  # gate and up projections
            check_float("dHg", f64(L.sparse_rows(L.plane(L.dh, 0), rows)), dH[0], prec, report)
            check_float("dHu", f64(L.sparse_rows(L.plane(L.dh, 1), rows)), dH[1], prec, report)
        else:
            check_float("dH", f64(L.sparse_rows(L.dh, rows)), dH, prec, report)
        if not (L.fuse_top1 and not sw):  # top-1 GeLU: dx straight from the product
            check_float("dXp", f64(L.dxp[rows.long()]), dXp, prec, report)
        check_float("dx", f64(L.dx[torch.from_numpy(toks).cuda()]), O.backward_tokens(toks),
                    prec, report)
        wr, wc = wgrad_samples(cfg, r, case.n_wgrad)
        got = f64(L.dW2[torch.from_numpy(wr).cuda()][:, torch.from_numpy(wc).cuda()])
        check_float("dW2", got, O.dW2_block(wr, wc), prec, report)
        # dW1 [d, E*f]: rows = model dims, cols = expert hidden units
        got1 = f64(L.dW1[torch.from_numpy(wc).cuda()][:, torch.from_numpy(wr).cuda()])
        check_float("dW1", got1, O.dW1_block(wc, wr), prec, report)
        if sw:
            got3 = f64(L.dW3[torch.from_numpy(wc).cuda()][:, torch.from_numpy(wr).cuda()])
            check_float("dW3", got3, O.dW3_block(wc, wr), prec, report)
        # gate backward on the sampled tokens: the oracle differentiates its
        # own stored Yp, the GPU its own
        # (Yp rows are in assignment order: token toks[i]'s k rows at i*k + j)
        want_dl = orc.route_backward(inp["logits"][toks], cfg.k,
                                     r["expert_idx"].reshape(cfg.T, cfg.k)[toks].reshape(-1),
                                     inp["dy"].values[toks], Yp, cfg.renorm)
        got_dl = L.dlogits[torch.from_numpy(toks).cuda()].cpu().numpy().astype(np.float64)
        check_float("dlogits", got_dl, want_dl, prec, report)
        empty = np.nonzero(r["counts"] == 0)[0]
        for e in empty:  # experts without tokens: exactly zero weight gradients
            assert torch.count_nonzero(L.dW2[e * cfg.f:(e + 1) * cfg.f]).item() == 0
            assert torch.count_nonzero(L.dW1[:, e * cfg.f:(e + 1) * cfg.f]).item() == 0
            if sw:
                assert torch.count_nonzero(L.dW3[:, e * cfg.f:(e + 1) * cfg.f]).item() == 0
    _say(f"[parity] {cfg.name} ok; max|d|/max|o|: " +
         ", ".join(f"{k}={v:.2e}" for k, v in report.items()))
    return L, dev, inp


# ------------------------------------------------------------ small cases

def _small(name, **kw):
    base = dict(T=1000, d=256, E=5, f=384, k=2, act="gelu", dtype="bf16", backward=True)
    base.update(kw)
    return synth.LayerConfig(name, **base)


def _assign_logits(T, E, experts):
    """Logits that send token t to experts[t] (top-1): 8 for the pick, 0 else."""
    lg = np.zeros((T, E), np.float32)
    lg[np.arange(T), experts] = 8.0
    return lg


SMALL = {
    # several tiles and a ragged tail; F = 3 (odd: one block per SDD tile)
    "ragged_bf16": Case(_small("ragged_bf16")),
    "ragged_f32": Case(_small("ragged_f32", dtype="f32", x_std=0.5)),
    # F = 2 (pairs of blocks per SDD tile), N not a multiple of 256
    "pairs_bf16": Case(_small("pairs_bf16", T=700, d=384, E=3, f=256, k=1)),
    "d_f_128": Case(_small("d_f_128", T=300, d=128, E=3, f=128, k=1)),
    "k_equals_E": Case(_small("k_equals_E", T=200, d=128, E=4, f=256, k=4)),
    "swiglu_small": Case(_small("swiglu_small", T=500, d=256, E=4, f=256, k=2, act="swiglu",
                                renorm=True, yp_dtype="f32", backward=False)),
    "swiglu_f32": Case(_small("swiglu_f32", T=300, d=128, E=3, f=256, k=2, act="swiglu",
                              dtype="f32", renorm=True, backward=False, x_std=0.5)),
    # SwiGLU training: F = 3 (a ragged column pair in the backward SDD), d = 384
    # (an absent N half in the two-set DSD and the DSTDs)
    "swiglu_train_bf16": Case(_small("swiglu_train_bf16", T=600, d=384, E=4, f=384, k=2,
                                     act="swiglu", renorm=True, yp_dtype="f32")),
    "swiglu_train_bf16_ypbf16": Case(_small("swiglu_train_bf16_ypbf16", T=500, d=256, E=3,
                                            f=256, k=1, act="swiglu")),
    "swiglu_train_f32": Case(_small("swiglu_train_f32", T=300, d=128, E=3, f=256, k=2,
                                    act="swiglu", dtype="f32", renorm=True, x_std=0.5)),
    # rows of 128 or more 16-byte chunks, not a multiple of 128: the backward's
    # dy permutation keeps two chunks per lane in flight, with some lanes
    # holding one (bf16 d = 1152: 144 chunks; fp32 d = 640: 160 chunks)
    "long_rows_bf16": Case(_small("long_rows_bf16", T=300, d=1152, E=4, f=256, k=2)),
    "long_rows_yp_f32": Case(_small("long_rows_yp_f32", T=300, d=1152, E=3, f=128, k=2,
                                    renorm=True, yp_dtype="f32")),
    "long_rows_f32": Case(_small("long_rows_f32", T=200, d=640, E=3, f=128, k=1, dtype="f32",
                                 x_std=0.5)),
    # bins padded to 256 rows (every expert an even number of block rows)
    "bins256_bf16": Case(_small("bins256_bf16", bin_rows=256)),
    # bins of 64 rows in blocks of 64 rows: tiles of up to four block rows
    "bins64_bf16": Case(_small("bins64_bf16", bin_rows=64)),
    "bins64_f32": Case(_small("bins64_f32", T=700, d=256, E=6, f=256, k=2, dtype="f32",
                              x_std=0.5, bin_rows=64)),
    "bins64_swiglu": Case(_small("bins64_swiglu", T=600, d=384, E=4, f=384, k=2,
                                 act="swiglu", renorm=True, yp_dtype="f32", bin_rows=64)),
    "bins64_top1_bf16": Case(_small("bins64_top1_bf16", T=900, d=384, E=5, f=256, k=1,
                                    bin_rows=64)),
    "bins256_swiglu": Case(_small("bins256_swiglu", T=500, d=256, E=4, f=256, k=2,
                                  act="swiglu", renorm=True, yp_dtype="f32", bin_rows=256)),
}


def _edge_cases():
    cases = {}
    # an expert that receives no token (dW must be zero, DSTD writes zeros)
    cfg = _small("empty_expert", T=400, d=128, E=6, f=256, k=1)
    lg = np.random.default_rng(3).standard_normal((400, 6)).astype(np.float32)
    lg[:, 3] = -50.0
    cases["empty_expert"] = Case(cfg, logits=lg)
    cfg = _small("empty_expert_swiglu", T=400, d=128, E=6, f=256, k=2, act="swiglu", renorm=True)
    cases["empty_expert_swiglu"] = Case(cfg, logits=lg)
    # every token on one expert
    cfg = _small("one_expert", T=300, d=128, E=4, f=256, k=1)
    cases["one_expert"] = Case(cfg, logits=_assign_logits(300, 4, np.zeros(300, int)))
    # counts that are exact multiples of 128: no pad rows at all
    cfg = _small("no_padding", T=512, d=128, E=4, f=256, k=1)
    cases["no_padding"] = Case(cfg, logits=_assign_logits(512, 4, np.arange(512) // 128))
    # counts 1, 127, 128, 129
    ex = np.repeat(np.arange(4), [1, 127, 128, 129])
    cfg = _small("counts_1_127_128_129", T=385, d=128, E=4, f=128, k=1)
    cases["counts_1_127_128_129"] = Case(cfg, logits=_assign_logits(385, 4, ex))
    # more experts than lanes (several logits per lane in routing and the gate
    # backward), up to the 1024-expert limit, and the largest top-k
    cases["many_experts"] = Case(_small("many_experts", T=1500, d=128, E=300, f=128, k=3))
    cases["max_experts"] = Case(_small("max_experts", T=3000, d=128, E=1024, f=128, k=2,
                                       renorm=True), n_tokens=200, n_wgrad=64)
    cases["max_topk"] = Case(_small("max_topk", T=200, d=128, E=40, f=128, k=32, renorm=True))
    # bins of 64 rows: experts ending in tiles of 1, 2, 3 and 4 block rows of
    # 64, one expert of seven block rows (4 + 3), one without tokens
    ex = np.repeat(np.arange(6), [59, 125, 182, 256, 447, 0])
    cfg = _small("bins64_slots", T=1069, d=256, E=6, f=384, k=1, bin_rows=64)
    cases["bins64_slots"] = Case(cfg, logits=_assign_logits(1069, 6, ex))
    cfg = _small("bins64_slots_swiglu", T=1069, d=256, E=6, f=256, k=1, act="swiglu",
                 bin_rows=64)
    cases["bins64_slots_swiglu"] = Case(cfg, logits=_assign_logits(1069, 6, ex))
    # ties in the logits (lower id wins)
    cfg = _small("ties", T=256, d=128, E=8, f=128, k=2)
    lg = np.random.default_rng(4).integers(-2, 3, size=(256, 8)).astype(np.float32)
    cases["ties"] = Case(cfg, logits=lg)
    # long K walks with closed-form K-block indices: a block row of 2050
    # blocks (the DSD's K) ...
    cfg = _small("long_block_rows", T=200, d=128, E=1, f=128 * 2050, k=1)
    cases["long_block_rows"] = Case(cfg, n_tokens=16, n_wgrad=16)
    # ... and a block column of 2050 blocks (the DSTD's K)
    cfg = _small("long_block_cols", T=128 * 2049 + 5, d=128, E=1, f=128, k=1)
    cases["long_block_cols"] = Case(cfg, n_tokens=16, n_wgrad=16)
    return cases


EDGE = _edge_cases()


def _picks_logits(T, E, k, counts, seed):
    """Logits under which expert e receives exactly counts[e] of the T*k
    picks (every count at most T), each token k distinct experts, tokens in
    a seeded random order; the picks' logits are 8 - 2 j (+ noise) for slot
    j, every other logit lies in [-1, 1)."""
    counts = np.asarray(counts)
    assert counts.sum() == T * k and counts.max() <= T
    rng = np.random.default_rng(seed)
    flat = np.repeat(np.arange(E), counts)          # runs of at most T entries
    picks = flat.reshape(k, T).T                    # token t: flat[t], flat[t + T], ...
    picks = picks[rng.permutation(T)]
    lg = rng.uniform(-1.0, 1.0, size=(T, E)).astype(np.float32)
    for j in range(k):
        lg[np.arange(T), picks[:, j]] = 8.0 - 2.0 * j + rng.uniform(0, 0.5, T)
    return np.ascontiguousarray(lg)


# Tile groups of 4 and 8 row pairs (set from Tp_max and E), compared element
# by element: every expert ends in a half tile or a short last group (or
# both), and the DSTD column-pair groups hold fewer pairs than G at the end.
GROUPS = {
    # Tp_max 4480, E 4: G = 4.  Block rows 15, 11, 6, 3: groups 4+4 (half at
    # the end), 4+2 (half), 3, 2 (half); F = 9 (column-pair groups 4+1, a
    # single last column); d = 384 (an absent N half)
    "group4_gelu": (_small("group4_gelu", T=4096, d=384, E=4, f=1152, k=1),
                    [1800, 1300, 700, 296], 4),
    # Tp_max 8576, E 4: G = 8.  Block rows 27, 19, 13, 7 (all odd): groups
    # 8+6, 8+2, 7, 4, each ending in a half tile; F = 17
    "group8_gelu": (_small("group8_gelu", T=8192, d=256, E=4, f=2176, k=1),
                    [3400, 2400, 1600, 792], 8),
    # SwiGLU trained, top-2: Tp_max 16768, E 4: G = 8.  Block rows 47, 35,
    # 28, 20: groups 8+8+8 (half), 8+8+2 (half), 8+6, 8+2; the two-set DSD
    # and three DSTDs; F = 9
    "group8_swiglu_train": (_small("group8_swiglu_train", T=8192, d=128, E=4, f=1152, k=2,
                                   act="swiglu", renorm=True, yp_dtype="f32"),
                            [6000, 4400, 3500, 2484], 8),
}


def _bf16_draw(rng, shape, std):
    """Seeded N(0, std) values rounded to bf16 (host-side, round to nearest even)."""
    v = (rng.standard_normal(shape) * std).astype(np.float32)
    return synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(v)).reshape(shape)


@pytest.mark.parametrize("bin_rows", [128, 64])
@pytest.mark.parametrize("name", list(GROUPS))
def test_products_at_tile_groups(orc, name, bin_rows):
    """SDD, DSD and DSTD called directly on seeded operands shared with the
    oracle, on the topologies of the tile-group cases (groups of 4 and 8 row
    tiles with partial tiles and short last groups, column-pair groups with a
    short last group), in blocks of 128 rows and, over bins of 64, of 64 rows
    (tiles ending in 1, 2 or 3 of their 4 block rows): every output element
    against the oracle's block products, with every epilogue, operand layout
    and output form the layer uses at these shapes.  Only the accumulation
    (fp32 against fp64) and the final rounding differ between the two sides,
    so the bar applies as is."""
    from block_sparse_gemm_amd import bsg, layer
    cfg, counts, G = GROUPS[name]
    cfg = cfg.replace(bin_rows=bin_rows)
    BR = 64 if bin_rows == 64 else 128
    _say(f"[products] {name} T={cfg.T} d={cfg.d} E={cfg.E} f={cfg.f} k={cfg.k} act={cfg.act} "
         f"bin_rows={bin_rows}")
    lg = _picks_logits(cfg.T, cfg.E, cfg.k, counts, seed=31)
    L = layer.Layer(layer.Shape.of(cfg))
    bsg.route(torch.from_numpy(lg).cuda(), cfg.k, cfg.renorm, L.expert_idx, L.gate, L.dest_row,
              L.counts, L.bin_offsets, L.route_ws, bin_rows=bin_rows)
    bsg.build_topology(L.bin_offsets, cfg.E, cfg.f, L.Tp_max, L.topo)
    torch.cuda.synchronize()
    r = orc.route(lg, cfg.k, cfg.renorm, bin_rows)
    bo = r["bin_offsets"]
    assert np.array_equal(L.bin_offsets.cpu().numpy(), bo)
    assert L.topo.meta[2].item() == 0
    E, F, d, f = cfg.E, cfg.f // 128, cfg.d, cfg.f
    Tp, nnz, nnz_max = int(bo[E]), int(bo[E]) // BR * F, L.topo.nnz_max
    rng = np.random.default_rng(41)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda().to(torch.bfloat16)
    blocks_of = lambda t, planes=1: t.view(planes, nnz_max, BR, 128)[:, :nnz].float() \
        .cpu().double().numpy().reshape(planes * nnz, BR, 128)
    P = dict(block_rows=BR)
    report = {}

    def compare(label, got, want):
        check_float(label, got, want, "bf16", report)

    xp = _bf16_draw(rng, (L.Tp_max, d), 1.0)          # rows at or beyond Tp are not read
    W1 = _bf16_draw(rng, (d, E * f), 0.05)            # [d, E*f]
    W2 = _bf16_draw(rng, (E * f, d), 0.05)            # [E*f, d]
    sw = cfg.act == "swiglu"
    W3 = _bf16_draw(rng, (d, E * f), 0.05) if sw else None
    planes = 2 if sw else 1
    out = torch.zeros(planes * nnz_max * BR, 128, dtype=torch.bfloat16, device="cuda")
    aux = torch.zeros_like(out)
    # forward SDD, saving the backward's factor(s)
    if sw:
        bsg.sdd(dev(xp), dev(W1), d, L.topo, "silu_mul", out[:nnz_max * BR], b2=dev(W3),
                aux_out=aux)
        A, SQ = orc.sdd(xp, W1, d, bo, E, F, "silu_mul", b2=W3, want_aux=True, **P)
        torch.cuda.synchronize()
        compare("sdd A", blocks_of(out[:nnz_max * BR]), A)
        compare("sdd S, Q", blocks_of(aux, 2), SQ)
    else:
        bsg.sdd(dev(xp), dev(W1), d, L.topo, "gelu", out, aux_out=aux)
        A, Gp = orc.sdd(xp, W1, d, bo, E, F, "gelu", want_aux=True, **P)
        torch.cuda.synchronize()
        compare("sdd A", blocks_of(out), A)
        compare("sdd G", blocks_of(aux), Gp)
    # backward SDD: B transposed (W2 as stored), saved factor(s) in
    dyp = _bf16_draw(rng, (L.Tp_max, d), 1.0)
    saved = _bf16_draw(rng, (planes * nnz_max * BR, 128), 1.0)
    saved_used = saved.reshape(planes, nnz_max, BR, 128)[:, :nnz].reshape(-1)
    bsg.sdd(dev(dyp), dev(W2), d, L.topo, "silu_mul_bwd" if sw else "gelu_bwd", out,
            trans_b=True, aux_in=dev(saved))
    want = orc.sdd(dyp, W2, d, bo, E, F, "silu_mul_bwd" if sw else "gelu_bwd", trans_b=True,
                   aux_in=saved_used, **P)
    torch.cuda.synchronize()
    compare("sdd_bwd dH", blocks_of(out, planes), want)
    # DSD: W2 as stored, bf16 rows; and B transposed with fp32 rows (two sets for SwiGLU)
    blk = _bf16_draw(rng, (planes * nnz_max * BR, 128), 1.0)
    blk_used = blk.reshape(planes, nnz_max, BR, 128)[:, :nnz].reshape(planes * nnz, BR, 128)
    c16 = torch.zeros(L.Tp_max, d, dtype=torch.bfloat16, device="cuda")
    bsg.dsd(dev(blk[:nnz_max * BR]), L.topo, dev(W2), d, c16)
    want = orc.dsd(blk_used[:nnz], bo, E, F, W2, d, **P)
    torch.cuda.synchronize()
    compare("dsd", c16[:Tp].double().cpu().numpy(), want)
    c32 = torch.zeros(L.Tp_max, d, dtype=torch.float32, device="cuda")
    if sw:
        bsg.dsd(dev(blk[:nnz_max * BR]), L.topo, dev(W1), d, c32, trans_b=True,
                blocks2=dev(blk[nnz_max * BR:]), b2=dev(W3))
        want = orc.dsd(blk_used[:nnz], bo, E, F, W1, d, prec="f32", trans_b=True,
                       blocks2=blk_used[nnz:], b2=W3, **P)
    else:
        bsg.dsd(dev(blk), L.topo, dev(W1), d, c32, trans_b=True)
        want = orc.dsd(blk_used, bo, E, F, W1, d, prec="f32", trans_b=True, **P)
    torch.cuda.synchronize()
    compare("dsd (B transposed, fp32 rows)", c32[:Tp].double().cpu().numpy(), want)
    # DSTD through the transpose index, stored as is and transposed
    dm = torch.zeros(L.Tp_max, d, dtype=torch.bfloat16, device="cuda")
    dm[:Tp] = dev(xp[:Tp])                                 # rows past Tp are never read
    want = orc.dstd(blk_used[:nnz], bo, E, F, xp[:Tp], d, **P)
    dW = torch.zeros(E * f, d, dtype=torch.bfloat16, device="cuda")
    dWt = torch.zeros(d, E * f, dtype=torch.bfloat16, device="cuda")
    bsg.dstd(dev(blk[:nnz_max * BR]), L.topo, dm, d, dW)
    bsg.dstd(dev(blk[:nnz_max * BR]), L.topo, dm, d, dWt, trans_c=True)
    torch.cuda.synchronize()
    compare("dstd", dW.double().cpu().numpy(), want)
    compare("dstd (transposed)", dWt.double().cpu().numpy().T, want)
    _say(f"[products] {name} bin_rows={bin_rows} ok; max|d|/max|o|: " +
         ", ".join(f"{k}={v:.2e}" for k, v in report.items()))


# DSD with a split last round (a tile walks >= 32 K-blocks).  few_tiles:
# 16 tiles (d = 384: an absent N half in every second column tile, a half row
# pair), all of them in the split round, 8 shares each; the same over bins of
# 64 (64-row blocks, a tile with one block row); two_sets: the SwiGLU input
# gradient (2 x 16 K-blocks), 10 tiles with two half row pairs; tail_of_many:
# 280 tiles on the 256 CUs of an MI355X, 256 whole and the last 24 (the last
# group of 3 row pairs, one of them half) split 8 ways.
SPLIT = {
    "few_tiles": (_small("split_few", T=1536, d=384, E=4, f=4096, k=1),
                  [650, 450, 300, 136], 128),
    "few_tiles_bins64": (_small("split_few64", T=1536, d=384, E=4, f=4096, k=1),
                         [650, 450, 300, 136], 64),
    "two_sets": (_small("split_two", T=1024, d=256, E=4, f=2048, k=2, act="swiglu"),
                 [800, 600, 400, 248], 128),
    "tail_of_many": (_small("split_tail", T=8832, d=2048, E=1, f=4096, k=1), [8832], 128),
}


@pytest.mark.parametrize("name", list(SPLIT))
def test_dsd_split_last_round(orc, name):
    """bsg_dsd with a workspace: the last round's tiles are cut into K-segments
    whose fp32 partial sums a second launch adds in segment order.  Against
    the oracle (every element, or for tail_of_many 64 sampled rows, half of
    them in the split tiles, from the product's definition in fp64); against
    the same product without the workspace (only the split tiles' fp32 sums
    associate differently); and bit-identical on a second run."""
    from block_sparse_gemm_amd import bsg, layer
    cfg, counts, bin_rows = SPLIT[name]
    cfg = cfg.replace(bin_rows=bin_rows)
    BR = 64 if bin_rows == 64 else 128
    _say(f"[split] {name} T={cfg.T} d={cfg.d} E={cfg.E} f={cfg.f} k={cfg.k} act={cfg.act} "
         f"bin_rows={bin_rows}")
    lg = _picks_logits(cfg.T, cfg.E, cfg.k, counts, seed=37)
    L = layer.Layer(layer.Shape.of(cfg.replace(backward=False)))
    bsg.route(torch.from_numpy(lg).cuda(), cfg.k, cfg.renorm, L.expert_idx, L.gate, L.dest_row,
              L.counts, L.bin_offsets, L.route_ws, bin_rows=bin_rows)
    bsg.build_topology(L.bin_offsets, cfg.E, cfg.f, L.Tp_max, L.topo)
    torch.cuda.synchronize()
    bo = orc.route(lg, cfg.k, cfg.renorm, bin_rows)["bin_offsets"]
    assert np.array_equal(L.bin_offsets.cpu().numpy(), bo)
    E, F, d, f = cfg.E, cfg.f // 128, cfg.d, cfg.f
    Tp, nnz, nnz_max = int(bo[E]), int(bo[E]) // BR * F, L.topo.nnz_max
    sw = cfg.act == "swiglu"
    planes = 2 if sw else 1
    rng = np.random.default_rng(43)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda().to(torch.bfloat16)
    blk = _bf16_draw(rng, (planes * nnz_max * BR, 128), 1.0)
    blk_used = blk.reshape(planes, nnz_max, BR, 128)[:, :nnz].reshape(planes * nnz, BR, 128)
    W = _bf16_draw(rng, (d, E * f), 0.05)           # W1 [d, E*f]: B transposed
    W3 = _bf16_draw(rng, (d, E * f), 0.05) if sw else None
    ws = torch.empty(bsg.dsd_workspace_bytes() // 4, dtype=torch.float32, device="cuda")
    a_dev = dev(blk)
    w_dev, w3_dev = dev(W), (dev(W3) if sw else None)
    kw = dict(trans_b=True)
    if sw:
        kw.update(blocks2=a_dev[nnz_max * BR:], b2=w3_dev)
    a0 = a_dev[:nnz_max * BR]
    outs = {}
    for c_dtype in (torch.float32, torch.bfloat16):
        ref = torch.zeros(L.Tp_max, d, dtype=c_dtype, device="cuda")
        got = torch.zeros_like(ref)
        again = torch.zeros_like(ref)
        bsg.dsd(a0, L.topo, w_dev, d, ref, **kw)
        bsg.dsd(a0, L.topo, w_dev, d, got, workspace=ws, **kw)
        bsg.dsd(a0, L.topo, w_dev, d, again, workspace=ws, **kw)
        torch.cuda.synchronize()
        outs[c_dtype] = (ref[:Tp].double().cpu().numpy(), got[:Tp].double().cpu().numpy())
        assert torch.equal(got, again), "split DSD not deterministic"
    report = {}
    got32 = outs[torch.float32][1]
    if not sw:
        # B as stored ([E*f, d], W2's layout) holding the same values: the same
        # products in the same order, so the same bits
        stored = torch.zeros(L.Tp_max, d, dtype=torch.float32, device="cuda")
        bsg.dsd(a0, L.topo, dev(np.ascontiguousarray(W.T)), d, stored, workspace=ws)
        torch.cuda.synchronize()
        assert np.array_equal(stored[:Tp].double().cpu().numpy(), got32), \
            "split DSD: B as stored differs from B transposed"
    if name != "tail_of_many":
        want = orc.dsd(blk_used[:nnz], bo, E, F, W, d, prec="f32", trans_b=True,
                       block_rows=BR, **(dict(blocks2=blk_used[nnz:], b2=W3) if sw else {}))
        check_float("split dsd fp32 rows", got32, want, "bf16", report)
        want16 = orc.dsd(blk_used[:nnz], bo, E, F, W, d, trans_b=True, block_rows=BR,
                         **(dict(blocks2=blk_used[nnz:], b2=W3) if sw else {}))
        check_float("split dsd bf16 rows", outs[torch.bfloat16][1], want16, "bf16", report)
    else:
        # rows: 32 from the split tiles (the last 3 row pairs), 32 from the rest
        split_rows = rng.choice(np.arange(Tp - 3 * 256 + 128, Tp), 32, replace=False)
        other = rng.choice(np.arange(0, Tp - 3 * 256), 32, replace=False)
        rows = np.sort(np.concatenate([split_rows, other]))
        # row r of the product: the F blocks of its block row (block id rb * F + j
        # in BCSR order, one expert) against W^T
        Wt = W.T.astype(np.float64)
        want = np.stack([np.concatenate([blk[((r // BR) * F + j) * BR + r % BR] for j in range(F)])
                         .astype(np.float64) @ Wt for r in rows])
        check_float("split dsd sampled rows", got32[rows], want, "bf16", report)
    # the split changes only how the tail tiles' fp32 sums associate
    ref32 = outs[torch.float32][0]
    rel = np.max(np.abs(got32 - ref32)) / max(np.max(np.abs(ref32)), 1e-30)
    assert rel <= 1e-5, f"split vs whole tiles (fp32): {rel}"
    r16, g16 = outs[torch.bfloat16]
    assert np.all(np.abs(g16 - r16) <= 2.0 ** -7 * np.maximum(1.0, np.abs(r16)))
    report["split vs whole (fp32)"] = float(rel)
    _say(f"[split] {name} ok; " + ", ".join(f"{k}={v:.2e}" for k, v in report.items()))


@pytest.mark.parametrize("bin_rows", [128, 64])
def test_sdd_split_last_round(orc, bin_rows):
    """An SDD launch of 288 tiles on the 256 CUs of an MI355X: the last 32
    (the last group: one full row tile, one holding a single block row, each
    x 16 column pairs) run as two half tiles each, the second half of the
    single-block-row tile as nothing.  Every element of A, G (forward with
    GeLU' kept) and dH (backward) against the oracle."""
    from block_sparse_gemm_amd import bsg, layer
    cfg = _small("split_sdd", T=4408, d=256, E=2, f=4096, k=1, bin_rows=bin_rows)
    counts = [2048, 2360]
    BR = 64 if bin_rows == 64 else 128
    _say(f"[sdd split] T={cfg.T} d={cfg.d} E={cfg.E} f={cfg.f} bin_rows={bin_rows}")
    lg = _picks_logits(cfg.T, cfg.E, cfg.k, counts, seed=47)
    L = layer.Layer(layer.Shape.of(cfg))
    bsg.route(torch.from_numpy(lg).cuda(), cfg.k, cfg.renorm, L.expert_idx, L.gate, L.dest_row,
              L.counts, L.bin_offsets, L.route_ws, bin_rows=bin_rows)
    bsg.build_topology(L.bin_offsets, cfg.E, cfg.f, L.Tp_max, L.topo)
    torch.cuda.synchronize()
    bo = orc.route(lg, cfg.k, cfg.renorm, bin_rows)["bin_offsets"]
    assert np.array_equal(L.bin_offsets.cpu().numpy(), bo)
    assert L.topo.meta[3].item() * (cfg.f // 256) == 288      # row tiles x column pairs
    E, F, d = cfg.E, cfg.f // 128, cfg.d
    nnz, nnz_max = int(bo[E]) // BR * F, L.topo.nnz_max
    rng = np.random.default_rng(53)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda().to(torch.bfloat16)
    blocks_of = lambda t: t.view(nnz_max, BR, 128)[:nnz].float().cpu().double().numpy()
    P = dict(block_rows=BR)
    report = {}
    xp = _bf16_draw(rng, (L.Tp_max, d), 1.0)
    W1 = _bf16_draw(rng, (d, E * cfg.f), 0.05)
    W2 = _bf16_draw(rng, (E * cfg.f, d), 0.05)
    out = torch.zeros(nnz_max * BR, 128, dtype=torch.bfloat16, device="cuda")
    aux = torch.zeros_like(out)
    bsg.sdd(dev(xp), dev(W1), d, L.topo, "gelu", out, aux_out=aux)
    A, Gp = orc.sdd(xp, W1, d, bo, E, F, "gelu", want_aux=True, **P)
    torch.cuda.synchronize()
    check_float("sdd A", blocks_of(out), A, "bf16", report)
    check_float("sdd G", blocks_of(aux), Gp, "bf16", report)
    dyp = _bf16_draw(rng, (L.Tp_max, d), 1.0)
    saved = _bf16_draw(rng, (nnz_max * BR, 128), 1.0)
    bsg.sdd(dev(dyp), dev(W2), d, L.topo, "gelu_bwd", out, trans_b=True, aux_in=dev(saved))
    want = orc.sdd(dyp, W2, d, bo, E, F, "gelu_bwd", trans_b=True,
                   aux_in=saved.reshape(nnz_max, BR, 128)[:nnz].reshape(-1), **P)
    torch.cuda.synchronize()
    check_float("sdd_bwd dH", blocks_of(out), want, "bf16", report)
    # the SwiGLU backward product on the same split: two saved planes in, two out
    out2 = torch.zeros(2 * nnz_max * BR, 128, dtype=torch.bfloat16, device="cuda")
    saved2 = _bf16_draw(rng, (2 * nnz_max * BR, 128), 1.0)
    bsg.sdd(dev(dyp), dev(W2), d, L.topo, "silu_mul_bwd", out2, trans_b=True,
            aux_in=dev(saved2))
    want = orc.sdd(dyp, W2, d, bo, E, F, "silu_mul_bwd", trans_b=True,
                   aux_in=saved2.reshape(2, nnz_max, BR, 128)[:, :nnz].reshape(-1), **P)
    torch.cuda.synchronize()
    got2 = out2.view(2, nnz_max, BR, 128)[:, :nnz].float().cpu().double().numpy()
    check_float("sdd_bwd (SwiGLU) dHg, dHu", got2.reshape(2 * nnz, BR, 128), want, "bf16",
                report)
    _say(f"[sdd split] bin_rows={bin_rows} ok; max|d|/max|o|: " +
         ", ".join(f"{k}={v:.2e}" for k, v in report.items()))


@pytest.mark.parametrize("name", list(GROUPS))
def test_tile_groups_full(orc, name):
    """The whole layer at groups of 4 and 8 row pairs, every output element
    against the oracle (forward and backward) except the weight gradients,
    which are compared on sampled rows and columns here and on every element
    in test_products_at_tile_groups: a weight-gradient entry sums an
    expert's thousands of products of two stored bf16 intermediates (A and
    dYp, or x and dH) that each side rounds on its own, and one factor that
    rounds to the neighbouring bf16 value moves the sum by about 2^-7 of one
    product, independent of the sum's size (readings of the tolerance in the
    design notes)."""
    from block_sparse_gemm_amd import bsg
    cfg, counts, G = GROUPS[name]
    Tp_max = bsg.max_padded_rows(cfg.T, cfg.k, cfg.E)
    rpe = Tp_max // (256 * cfg.E)
    assert (8 if (rpe >= 8 and cfg.E <= 16) else 4 if rpe >= 4 else 2) == G
    blocks = [-(-c // 128) for c in counts]
    assert any(b % 2 for b in blocks)                       # half tiles
    assert any(((b + 1) // 2) % G for b in blocks)          # short last groups
    lg = _picks_logits(cfg.T, cfg.E, cfg.k, counts, seed=31)
    L, _, _ = check_case(orc, Case(cfg, logits=lg, n_wgrad=48))
    assert L.counts.cpu().numpy().tolist() == list(counts)


@pytest.mark.parametrize("name", list(SMALL))
def test_small(orc, name):
    check_case(orc, SMALL[name])


@pytest.mark.parametrize("name", list(EDGE))
def test_edge(orc, name):
    check_case(orc, EDGE[name])


def test_deterministic(orc):
    """No atomics in the float path: two runs give bitwise identical outputs."""
    cfg = _small("determinism", T=700, d=256, E=5, f=256, k=2)
    inp = synth.make_inputs(cfg, 5)
    L1, _ = run_gpu(cfg, inp)
    L2, _ = run_gpu(cfg, inp)
    for name in ("y", "dx", "dW1", "dW2", "act", "dest_row"):
        assert torch.equal(getattr(L1, name), getattr(L2, name)), name


_TOPO_KEYS = ("row_ptr", "col_idx", "row_idx", "col_ptr", "trans_idx", "row_tiles",
              "expert_order", "meta")


@pytest.mark.parametrize("T,E,k,ws_offset,dtype", [
    (70000, 64, 2, 0, "bf16"),    # more than 1024 chunks: the count matrix is scanned first
    (20000, 1024, 1, 0, "bf16"),  # more than 65536 counts, the most experts
    (3000, 64, 2, 4, "f32"),      # a workspace off the 16-byte grid: counts summed one by one
    (65536, 2, 1, 0, "bf16"),     # 1024 chunks, two experts: the largest self-summed routing
    (1000, 8, 3, 0, "f32"),       # 4-count vectors of a power-of-two expert count
    (2000, 40, 32, 0, "bf16"),    # top-32: two chunks a placing workgroup at most
])
def test_route_topology_launch_paths(orc, T, E, k, ws_offset, dtype):
    """route + topology, and route + permutation (+ topology), in the
    routing's own launches equal route, permute_pad and build_topology
    called one by one, bit for bit, and all equal the oracle, on each of the
    placement's ways of forming the counts (scanned first, summed as
    vectors, summed one by one)."""
    from block_sparse_gemm_amd import bsg, layer
    _say(f"[parity] route_topology T={T} E={E} k={k} ws_offset={ws_offset} dtype={dtype}")
    f, d = 256, 128
    rng = np.random.default_rng(T + E)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    lg[:, 0] += 0.75  # mild skew
    xt = synth._draw(rng, (T, d), 1.0, dtype)
    r = orc.route(lg, k, False, 128)
    t = orc.topology(r["bin_offsets"], E, f // 128, 128)
    Tp = int(r["bin_offsets"][E])
    Tp_max = bsg.max_padded_rows(T, k, E)
    logits = torch.from_numpy(lg).cuda()
    x = layer.from_numpy(xt, dtype)
    i32 = dict(dtype=torch.int32, device="cuda")
    nbytes = bsg.route_workspace_bytes(T, k, E)
    outs = {}
    for mode in ("topology", "permute", "permute_no_topology", "separate"):
        o = dict(expert_idx=torch.full((T * k,), -7, **i32),
                 gate=torch.zeros(T * k, dtype=torch.float32, device="cuda"),
                 dest_row=torch.full((T * k,), -7, **i32), counts=torch.full((E,), -7, **i32),
                 bin_offsets=torch.full((E + 1,), -7, **i32),
                 row_src=torch.full((Tp_max,), -7, **i32),
                 xp=torch.full((Tp_max, d), 3.0, dtype=x.dtype, device="cuda"))
        ws = torch.full((nbytes + 16,), 0xAB, dtype=torch.uint8, device="cuda")
        ws = ws[ws_offset:ws_offset + nbytes]
        topo = bsg.Topology(Tp_max, E, f)
        for key in _TOPO_KEYS:
            getattr(topo, key).fill_(-7)
        if mode == "topology":
            bsg.route_topology(logits, k, False, o["expert_idx"], o["gate"], o["dest_row"],
                               o["counts"], o["bin_offsets"], ws, f, Tp_max, topo)
        elif mode.startswith("permute"):
            tp = topo if mode == "permute" else None
            bsg.route_permute_topology(logits, k, False, o["expert_idx"], o["gate"],
                                       o["dest_row"], o["counts"], o["bin_offsets"], ws, x,
                                       Tp_max, o["row_src"], o["xp"], f, tp)
        else:
            bsg.route(logits, k, False, o["expert_idx"], o["gate"], o["dest_row"], o["counts"],
                      o["bin_offsets"], ws)
            bsg.permute_pad(x, k, o["dest_row"], None, o["counts"], o["bin_offsets"], E, Tp_max,
                            o["row_src"], o["xp"])
            bsg.build_topology(o["bin_offsets"], E, f, Tp_max, topo)
        torch.cuda.synchronize()
        o = {key: v.cpu() for key, v in o.items()}
        o.update({key: getattr(topo, key).cpu() for key in _TOPO_KEYS})
        outs[mode] = o
    sep = outs["separate"]
    for mode, o in outs.items():
        keys = list(o)
        if mode == "topology":
            keys = [kk for kk in keys if kk not in ("row_src", "xp")]
        if mode == "permute_no_topology":
            keys = [kk for kk in keys if kk not in _TOPO_KEYS]
        for key in keys:
            assert torch.equal(o[key], sep[key]), (mode, key)
    o = {key: v.numpy() for key, v in sep.items() if key != "xp"}
    for key in ("expert_idx", "dest_row", "counts", "bin_offsets"):
        assert np.array_equal(o[key], r[key]), key
    assert np.array_equal(o["row_src"][:Tp], r["row_src"]), "row_src"
    xp_want = orc.permute_pad(xt.values, k, r["dest_row"], Tp, prec=dtype)
    assert np.array_equal(layer.to_numpy_f64(sep["xp"][:Tp]), xp_want), "xp"
    nnz, R = t["nnz"], Tp // 128
    assert o["meta"][0] == nnz and o["meta"][1] == R and o["meta"][2] == 0
    assert np.array_equal(o["row_ptr"][:R + 1], t["row_ptr"])
    for key in ("col_idx", "row_idx", "trans_idx"):
        assert np.array_equal(o[key][:nnz], t[key]), key
    assert np.array_equal(o["col_ptr"], t["col_ptr"])


# ------------------------------------------------------ full-size workloads

FULL = {
    "tiny": Case(synth.CONFIGS["tiny"]),
    "moe_xs": Case(synth.CONFIGS["moe_xs"], n_tokens=96),
    "moe_small": Case(synth.CONFIGS["moe_small"], n_tokens=64, n_wgrad=24),
    "mixtral": Case(synth.CONFIGS["mixtral"], n_tokens=12),
    "mixtral_train": Case(synth.CONFIGS["mixtral_train"], n_tokens=8, n_wgrad=8),
    "moe_xs_bins64": Case(synth.CONFIGS["moe_xs"].replace(name="moe_xs_bins64", bin_rows=64),
                          n_tokens=96),
    "moe_small_bins64": Case(synth.CONFIGS["moe_small"].replace(name="moe_small_bins64",
                                                                bin_rows=64),
                             n_tokens=48, n_wgrad=16),
    "moe_small_bins256": Case(synth.CONFIGS["moe_small"].replace(name="moe_small_bins256",
                                                                 bin_rows=256),
                              n_tokens=48, n_wgrad=16),
    "skew": Case(synth.CONFIGS["skew"], n_tokens=32, n_wgrad=16),
}


@pytest.mark.parametrize("name", list(FULL))
def test_full_size(orc, name):
    check_case(orc, FULL[name])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_permute_pad_scaled_exact(orc, dtype):
    """The scaled permutation rounds the exact product once: bit-exact
    against the oracle when both get the same (seeded) scale."""
    from block_sparse_gemm_amd import bsg, layer
    cfg = _small("scaled", T=900, d=384, E=7, f=128, k=3, dtype=dtype)
    inp = synth.make_inputs(cfg, 9, weights=False)
    rng = np.random.default_rng(11)
    scale = (rng.standard_normal(cfg.T * cfg.k) * 0.3).astype(np.float32)
    r = orc.route(inp["logits"], cfg.k)
    Tp = int(r["bin_offsets"][cfg.E])
    Tp_max = bsg.max_padded_rows(cfg.T, cfg.k, cfg.E)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    x = layer.from_numpy(inp["x"], dtype)
    xp = torch.full((Tp_max, cfg.d), 7.0, dtype=x.dtype, device="cuda")
    row_src = torch.full((Tp_max,), 99, dtype=torch.int32, device="cuda")
    bsg.permute_pad(x, cfg.k, dev(r["dest_row"]), dev(scale), dev(r["counts"]),
                    dev(r["bin_offsets"]), cfg.E, Tp_max, row_src, xp)
    torch.cuda.synchronize()
    want = orc.permute_pad(inp["x"].values, cfg.k, r["dest_row"], Tp, scale=scale, prec=dtype)
    assert np.array_equal(layer.to_numpy_f64(xp[:Tp]), want)
    assert np.array_equal(row_src[:Tp].cpu().numpy(), r["row_src"])
    # rows at and beyond Tp are untouched
    assert torch.all(xp[Tp:] == 7.0).item() and torch.all(row_src[Tp:] == 99).item()


def test_standalone_gate_backward_and_scaled_permute(orc):
    """The layer runs the fused dy permutation + gate backward; the two
    separate calls it replaces must give the same results: the scaled copy
    bit for bit, dlogits against the oracle."""
    from block_sparse_gemm_amd import bsg, layer
    cfg = _small("standalone_bwd", T=700, d=384, E=6, f=256, k=2, renorm=True)
    inp = synth.make_inputs(cfg, 13)
    L, dev = run_gpu(cfg, inp)
    dyp = torch.full_like(L.dyp, 3.0)
    row_src = torch.full_like(L.row_src_b, 7)
    dlogits = torch.full_like(L.dlogits, 5.0)
    bsg.permute_pad(dev["dy"], cfg.k, L.dest_row, L.gate, L.counts, L.bin_offsets, cfg.E,
                    L.Tp_max, row_src, dyp)
    bsg.route_backward(dev["logits"], cfg.k, cfg.renorm, L.expert_idx, L.dest_row, dev["dy"],
                       L.yp, dlogits)
    torch.cuda.synchronize()
    Tp = int(L.bin_offsets[-1].item())
    assert torch.equal(dyp[:Tp], L.dyp[:Tp])
    assert torch.equal(row_src[:Tp], L.row_src_b[:Tp])
    r = orc.route(inp["logits"], cfg.k, cfg.renorm)
    yp_rows = layer.to_numpy_f64(L.yp[torch.from_numpy(r["dest_row"]).cuda().long()])
    want = orc.route_backward(inp["logits"], cfg.k, r["expert_idx"], inp["dy"].values, yp_rows,
                              cfg.renorm)
    report = {}
    check_float("dlogits (standalone)", dlogits.cpu().numpy(), want, "bf16", report)
    check_float("dlogits (fused)", L.dlogits.cpu().numpy(), want, "bf16", report)


def test_permute_pad_never_writes_past_tp_max(orc):
    """Bins from a 256-row routing given to a buffer sized for 128-row bins:
    the copy writes nothing at or beyond Tp_max (sentinel rows inside the
    same allocation stay untouched)."""
    from block_sparse_gemm_amd import bsg, layer
    cfg = _small("clamp", T=300, d=128, E=7, f=128, k=2)
    inp = synth.make_inputs(cfg, 21, weights=False)
    r = orc.route(inp["logits"], cfg.k, False, 256)
    Tp128 = bsg.max_padded_rows(cfg.T, cfg.k, cfg.E, 128)
    assert int(r["bin_offsets"][cfg.E]) > Tp128  # the routing overruns the buffer
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    x = layer.from_numpy(inp["x"], "bf16")
    big = torch.full((Tp128 + 1024, cfg.d), 9.0, dtype=torch.bfloat16, device="cuda")
    row_src = torch.full((Tp128 + 1024,), 77, dtype=torch.int32, device="cuda")
    bsg.permute_pad(x, cfg.k, dev(r["dest_row"]), None, dev(r["counts"]),
                    dev(r["bin_offsets"]), cfg.E, Tp128, row_src[:Tp128], big[:Tp128])
    torch.cuda.synchronize()
    assert torch.all(big[Tp128:] == 9.0)
    assert torch.all(row_src[Tp128:] == 77)


@pytest.mark.parametrize("bwd", [False, True])
def test_top1_fused_combine_is_bit_identical(bwd):
    """The top-1 layer's combine inside the DSD epilogue gives the same bits
    as the separate DSD + unpermute_combine calls, forward and backward."""
    from block_sparse_gemm_amd import layer
    cfg = _small("fused_top1", T=900, d=384, E=5, f=256, k=1, backward=bwd)
    inp = synth.make_inputs(cfg, 17)
    outs = []
    for fuse in (True, False):
        L = layer.Layer(layer.Shape.of(cfg))
        assert L.fuse_top1
        L.fuse_top1 = fuse
        up = lambda key: layer.from_numpy(inp[key], cfg.dtype) if key in inp else None
        W1, W2 = up("W1"), up("W2")
        L.forward(up("x"), torch.from_numpy(inp["logits"]).cuda(), W1, W2)
        if bwd:
            L.backward(up("dy"), W1, W2)
        torch.cuda.synchronize()
        outs.append((L.y.clone(), L.yp.clone(), L.dx.clone() if bwd else None))
    assert torch.equal(outs[0][0], outs[1][0])
    if bwd:  # a forward-only top-1 layer writes no Yp
        assert torch.equal(outs[0][1], outs[1][1])
        assert torch.equal(outs[0][2], outs[1][2])


@pytest.mark.parametrize("act", ["gelu", "swiglu"])
def test_two_stream_schedule_gives_the_same_bits(act):
    """The backward with the weight gradients on a second stream gives the
    same bits as the one-stream order (every kernel is deterministic), also
    when it is run several times in a row."""
    from block_sparse_gemm_amd import layer
    kw = dict(act="swiglu", renorm=True, yp_dtype="f32") if act == "swiglu" else {}
    cfg = _small("two_streams", T=800, d=256, E=5, f=256, k=2, **kw)
    inp = synth.make_inputs(cfg, 23)
    up = lambda key: layer.from_numpy(inp[key], cfg.dtype) if key in inp else None
    x, W1, W2, W3, dy = up("x"), up("W1"), up("W2"), up("W3"), up("dy")
    logits = torch.from_numpy(inp["logits"]).cuda()
    names = ("y", "dx", "dW1", "dW2", "dlogits") + (("dW3",) if act == "swiglu" else ())
    results = []
    for overlap in (False, True):
        L = layer.Layer(layer.Shape.of(cfg))
        L.overlap = overlap
        for _ in range(3):
            L.step(x, logits, W1, W2, W3, dy)
        torch.cuda.synchronize()
        results.append({n: getattr(L, n).clone() for n in names})
    for n in names:
        assert torch.equal(results[0][n], results[1][n]), n


@pytest.mark.parametrize("act", ["gelu", "swiglu"])
def test_layer_reuse_across_routings(act):
    """One Layer called on two different routings in turn (A, B, A: other bin
    sizes, padded row counts and half tiles) gives, call by call, the same bits
    as a freshly allocated Layer on the same inputs: nothing a previous call
    left in the reused buffers reaches a result."""
    from block_sparse_gemm_amd import layer
    if act == "gelu":
        cfg = _small("reuse_gelu", T=900, d=256, E=6, f=256, k=2)
    else:
        cfg = _small("reuse_swiglu", T=700, d=256, E=4, f=256, k=2, act="swiglu", renorm=True,
                     yp_dtype="f32")
    ins = [synth.make_inputs(cfg, seed) for seed in (11, 12)]
    ins[1]["logits"] = ins[1]["logits"].copy()
    ins[1]["logits"][:, 0] += 2.0  # expert 0 takes most picks: other bins than routing A
    s = layer.Shape.of(cfg)
    names = ["y", "dx", "dW1", "dW2", "dlogits", "dest_row", "bin_offsets"]
    if act == "swiglu":
        names.append("dW3")

    def call(L, inp):
        up = lambda key: layer.from_numpy(inp[key], cfg.dtype) if key in inp else None
        x, W1, W2, W3, dy = up("x"), up("W1"), up("W2"), up("W3"), up("dy")
        L.forward(x, torch.from_numpy(inp["logits"]).cuda(), W1, W2, W3)
        L.backward(dy, W1, W2, W3)
        torch.cuda.synchronize()
        return {n: getattr(L, n).clone() for n in names}

    _say(f"[parity] layer reuse across routings, {act}")
    shared = layer.Layer(s)
    order = (0, 1, 0)
    got = [call(shared, ins[i]) for i in order]
    want = [call(layer.Layer(s), ins[i]) for i in order]
    assert not torch.equal(got[0]["bin_offsets"], got[1]["bin_offsets"]), "routings A and B differ"
    for c, (g, w) in enumerate(zip(got, want)):
        for n in names:
            assert torch.equal(g[n], w[n]), f"call {c}: {n}"
