"""Seeded synthetic inputs for the dropless-MoE expert layer.

This module only draws and stores inputs.  It holds none of the layer's
arithmetic (no routing, no products, no activation) so that the CPU oracle
and the GPU path can both consume exactly the same bytes without sharing any
computation.  Imported by the tests, the benchmark and the smoke entry point;
it never imports the GPU binding or the oracle.

Workloads (shapes follow the layer sizes named for the method; the pages print
no model shapes, so these are stand-ins for the training runs they measure):

=========  ======  ====  ===  =====  ===  ======  =====  =======
name        T       d     E    f      k    act     dtype  mode
=========  ======  ====  ===  =====  ===  ======  =====  =======
tiny        256     128   4    256    1    gelu    f32    fwd
moe_xs      16384   512   64   2048   1    gelu    bf16   fwd
moe_small   32768   768   64   3072   1    gelu    bf16   fwd+bwd
mixtral     8192    4096  8    14336  2    swiglu  bf16   fwd
skew        65536   1024  64   4096   2    gelu    bf16   fwd+bwd
=========  ======  ====  ===  =====  ===  ======  =====  =======

Draw order from ``numpy.random.default_rng(seed)``: logits [T,E] N(0,1) fp32,
then the per-expert logit bias (if any), then x [T,d], W1 [d,E*f], W3 [d,E*f]
(swiglu only), W2 [E*f,d], dy [T,d] N(0,1) (backward workloads only).  The
second parameter of N(mu, s) is the standard deviation.  Weights are
N(0,0.02); x is N(0,0.02) for ``tiny`` and N(0,1) for the rest.  bf16 inputs
are rounded from the fp32 draws with round-to-nearest-even.

Skewed load (``skew``): the experts are shuffled with ``rng.permutation(E)``;
the first 10 get +1.33 added to their logits and the last 6 get -1.0, so the
10 hottest experts receive about 75% of the assignments (the GPT-MoE skew
that George Lin's Blog reports in its FlexMoE section 2.1) and the starved
ones fall below 128 tokens.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

DTYPES = ("f32", "bf16")
ACTS = ("gelu", "swiglu")


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    name: str
    T: int
    d: int
    E: int
    f: int
    k: int
    act: str = "gelu"
    dtype: str = "bf16"
    backward: bool = False
    renorm: bool = False
    x_std: float = 1.0
    w_std: float = 0.02
    # logit recipe
    bias_std: float = 0.0          # per-expert N(0, bias_std) bias
    hot: int = 0                   # number of hot experts (skew recipe)
    hot_bias: float = 0.0
    starved: int = 0
    starved_bias: float = 0.0
    # Yp / dXp storage dtype ("bf16" or "f32"); f32 configs keep f32.
    yp_dtype: Optional[str] = None
    # expert bins padded to a multiple of bin_rows (128 = the block; 256 for
    # the block-size study)
    bin_rows: int = 128

    def __post_init__(self):
        assert self.dtype in DTYPES and self.act in ACTS
        assert 1 <= self.k <= self.E

    @property
    def yp(self) -> str:
        if self.dtype == "f32":
            return "f32"
        return self.yp_dtype or "bf16"

    @property
    def assignments(self) -> int:
        return self.T * self.k

    def replace(self, **kw) -> "LayerConfig":
        return dataclasses.replace(self, **kw)


CONFIGS = {
    "tiny": LayerConfig("tiny", T=256, d=128, E=4, f=256, k=1, act="gelu", dtype="f32",
                        x_std=0.02),
    "moe_xs": LayerConfig("moe_xs", T=16384, d=512, E=64, f=2048, k=1),
    "moe_small": LayerConfig("moe_small", T=32768, d=768, E=64, f=3072, k=1, backward=True,
                             bias_std=0.5),
    "mixtral": LayerConfig("mixtral", T=8192, d=4096, E=8, f=14336, k=2, act="swiglu",
                           renorm=True, yp_dtype="f32"),
    # the same layer trained: forward + backward of the SwiGLU experts
    "mixtral_train": LayerConfig("mixtral_train", T=8192, d=4096, E=8, f=14336, k=2,
                                 act="swiglu", renorm=True, yp_dtype="f32", backward=True),
    "skew": LayerConfig("skew", T=65536, d=1024, E=64, f=4096, k=2, backward=True,
                        hot=10, hot_bias=1.33, starved=6, starved_bias=-1.0),
}


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round finite fp32 values to bf16 (round to nearest, ties to even).

    Returns the raw 16-bit patterns as uint16."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to the fp32 values they encode (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass
class Tensor:
    """One input in its storage dtype: ``values`` are the exact fp32 values,
    ``bits`` the uint16 bf16 patterns (None for fp32 storage)."""
    values: np.ndarray
    bits: Optional[np.ndarray]

    @property
    def shape(self):
        return self.values.shape

    def storage(self) -> np.ndarray:
        """Array to upload to the device: uint16 bits for bf16, fp32 otherwise."""
        return self.bits if self.bits is not None else self.values


def _draw(rng, shape, std, dtype) -> Tensor:
    v = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        v *= np.float32(std)
    if dtype == "bf16":
        bits = f32_to_bf16_bits(v)
        return Tensor(bf16_bits_to_f32(bits).reshape(shape), bits.reshape(shape))
    return Tensor(v, None)


def make_logits(cfg: LayerConfig, rng) -> np.ndarray:
    logits = rng.standard_normal((cfg.T, cfg.E), dtype=np.float32)
    if cfg.bias_std > 0:
        bias = (rng.standard_normal(cfg.E, dtype=np.float32) * np.float32(cfg.bias_std))
        logits += bias[None, :]
    if cfg.hot or cfg.starved:
        perm = rng.permutation(cfg.E)
        bias = np.zeros(cfg.E, dtype=np.float32)
        if cfg.hot:
            bias[perm[: cfg.hot]] = np.float32(cfg.hot_bias)
        if cfg.starved:
            bias[perm[cfg.E - cfg.starved:]] = np.float32(cfg.starved_bias)
        logits += bias[None, :]
    return np.ascontiguousarray(logits)


def make_inputs(cfg: LayerConfig, seed: int = 0, weights: bool = True) -> dict:
    """All inputs of one layer call, drawn in the documented order.

    Keys: logits (fp32 [T,E]), x, W1, (W3), W2, (dy) as :class:`Tensor`.
    With ``weights=False`` only logits and x are drawn (the draws that follow
    are skipped, so the earlier ones are unchanged)."""
    rng = np.random.default_rng(seed)
    out = {"logits": make_logits(cfg, rng)}
    out["x"] = _draw(rng, (cfg.T, cfg.d), cfg.x_std, cfg.dtype)
    if not weights:
        return out
    out["W1"] = _draw(rng, (cfg.d, cfg.E * cfg.f), cfg.w_std, cfg.dtype)
    if cfg.act == "swiglu":
        out["W3"] = _draw(rng, (cfg.d, cfg.E * cfg.f), cfg.w_std, cfg.dtype)
    out["W2"] = _draw(rng, (cfg.E * cfg.f, cfg.d), cfg.w_std, cfg.dtype)
    if cfg.backward:
        out["dy"] = _draw(rng, (cfg.T, cfg.d), 1.0, cfg.dtype)
    return out


def sample_tokens(T: int, n: int, seed: int = 1) -> np.ndarray:
    """A sorted, seeded sample of ``n`` distinct token ids (always includes the
    first and the last token)."""
    n = min(n, T)
    rng = np.random.default_rng(seed)
    pick = rng.choice(T, size=n, replace=False)
    pick[0] = 0
    if n > 1:
        pick[1] = T - 1
    return np.unique(pick).astype(np.int64)
