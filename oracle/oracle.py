"""ctypes wrapper around the C oracle (``oracle/oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by the tests, ``__graft_entry__.smoke()``
and the benchmark's ``cpu_baseline`` leg, never by the product path.  It does
not import the GPU package.  Inputs are numpy arrays holding the exact values
of the stored inputs (bf16 inputs widened to fp32); float outputs come back as
fp64 arrays holding values already rounded to the requested storage precision.

See ``oracle.c`` for what each function computes and which passage of the
pages it follows.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle.so")
SRC_PATH = os.path.join(HERE, "oracle.c")

PREC = {"f64": 0, "f32": 1, "bf16": 2}
ACT = {"gelu": 0, "swiglu": 1}

_i64p = C.POINTER(C.c_int64)
_i32p = C.POINTER(C.c_int32)
_f32p = C.POINTER(C.c_float)
_f64p = C.POINTER(C.c_double)


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (-O2, OpenMP, no FP contraction)."""
    if not force and os.path.exists(LIB_PATH) and \
            os.path.getmtime(LIB_PATH) >= os.path.getmtime(SRC_PATH):
        return LIB_PATH
    tmp = LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-std=gnu11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-fPIC", "-shared", SRC_PATH, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


class _Layer(C.Structure):
    _fields_ = [
        ("T", C.c_int64), ("d", C.c_int), ("E", C.c_int), ("f", C.c_int), ("k", C.c_int),
        ("act", C.c_int), ("prec", C.c_int), ("prec_yp", C.c_int),
        ("x", _f32p), ("W1", _f32p), ("W3", _f32p), ("W2", _f32p), ("dy", _f32p),
        ("expert_idx", _i32p), ("gate", _f32p),
    ]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        L = C.CDLL(LIB_PATH)
        L.orc_round.restype = C.c_double
        L.orc_round.argtypes = [C.c_double, C.c_int]
        for name in ("orc_gelu", "orc_gelu_grad", "orc_silu", "orc_silu_grad"):
            getattr(L, name).restype = C.c_double
            getattr(L, name).argtypes = [C.c_double]
        L.orc_set_threads.argtypes = [C.c_int]
        L.orc_get_threads.restype = C.c_int
        L.orc_route.restype = C.c_int
        L.orc_route.argtypes = [_f32p, C.c_int64, C.c_int, C.c_int, C.c_int, C.c_int, _i32p, _f32p,
                                _i32p, _i32p, _i32p, _i32p, C.c_int64]
        L.orc_permute_pad.restype = C.c_int
        L.orc_permute_pad.argtypes = [_f32p, C.c_int64, C.c_int, C.c_int, _i32p, _f32p, C.c_int,
                                      C.c_int64, _f64p]
        L.orc_route_backward.restype = C.c_int
        L.orc_route_backward.argtypes = [_f32p, C.c_int64, C.c_int, C.c_int, C.c_int, _i32p,
                                         _f32p, _f64p, C.c_int, _f64p]
        L.orc_topology.restype = C.c_int64
        L.orc_topology.argtypes = [_i32p, C.c_int, C.c_int, C.c_int, _i32p, _i32p, _i32p, _i32p,
                                   _i32p]
        lp = C.POINTER(_Layer)
        L.orc_assign_forward.argtypes = [lp, _i64p, C.c_int64, _f64p, _f64p, _f64p, _f64p]
        L.orc_forward_tokens.argtypes = [lp, _i64p, C.c_int64, _f64p]
        L.orc_assign_backward.argtypes = [lp, _i64p, C.c_int64, _f64p, _f64p, _f64p, _f64p]
        L.orc_backward_tokens.argtypes = [lp, _i64p, C.c_int64, _f64p]
        for n in ("orc_dW2_block", "orc_dW1_block", "orc_dW3_block"):
            getattr(L, n).argtypes = [lp, _i64p, C.c_int64, _i64p, C.c_int64, _f64p]
        L.orc_sdd.restype = C.c_int64
        L.orc_sdd.argtypes = [_f32p, C.c_int64, _f32p, _f32p, C.c_int64, C.c_int, C.c_int, _i32p,
                              C.c_int, C.c_int, C.c_int, C.c_int, _f32p, C.c_int, _f64p, _f64p]
        L.orc_dsd.restype = C.c_int64
        L.orc_dsd.argtypes = [_f32p, _f32p, _i32p, C.c_int, C.c_int, C.c_int, _f32p, _f32p,
                              C.c_int64, C.c_int, C.c_int, C.c_int, _f64p]
        L.orc_dstd.restype = C.c_int
        L.orc_dstd.argtypes = [_f32p, _i32p, C.c_int, C.c_int, C.c_int, _f32p, C.c_int64,
                               C.c_int, C.c_int, _f64p]
        for n in ("orc_assign_forward", "orc_forward_tokens", "orc_assign_backward",
                  "orc_backward_tokens", "orc_dW2_block", "orc_dW1_block", "orc_dW3_block"):
            getattr(L, n).restype = C.c_int
        _lib = L
    return _lib


def _p(a, t):
    return a.ctypes.data_as(t) if a is not None else None


def _f32(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float32)


def set_threads(n: int) -> None:
    lib().orc_set_threads(int(n))


def get_threads() -> int:
    return int(lib().orc_get_threads())


def rd(v: float, prec: str) -> float:
    return lib().orc_round(float(v), PREC[prec])


def gelu(h: float) -> float:
    return lib().orc_gelu(float(h))


def gelu_grad(h: float) -> float:
    return lib().orc_gelu_grad(float(h))


def silu(z: float) -> float:
    return lib().orc_silu(float(z))


def silu_grad(z: float) -> float:
    return lib().orc_silu_grad(float(z))


def route(logits: np.ndarray, k: int, renorm: bool = False, bin_rows: int = 128) -> dict:
    """Top-k routing, gates, histogram, bins padded to a multiple of
    bin_rows, stable placement."""
    logits = _f32(logits)
    T, E = logits.shape
    out = {
        "expert_idx": np.zeros(T * k, np.int32),
        "gate": np.zeros(T * k, np.float32),
        "counts": np.zeros(E, np.int32),
        "bin_offsets": np.zeros(E + 1, np.int32),
        "dest_row": np.zeros(T * k, np.int32),
    }
    bound = T * k + (bin_rows - 1) * min(E, T * k) + bin_rows
    row_src = np.zeros(bound, np.int32)
    rc = lib().orc_route(_p(logits, _f32p), T, E, k, int(bool(renorm)), int(bin_rows),
                         _p(out["expert_idx"], _i32p), _p(out["gate"], _f32p),
                         _p(out["counts"], _i32p), _p(out["bin_offsets"], _i32p),
                         _p(out["dest_row"], _i32p), _p(row_src, _i32p), bound)
    if rc != 0:
        raise ValueError("orc_route rejected its arguments")
    out["row_src"] = row_src[: int(out["bin_offsets"][E])].copy()
    return out


def route_backward(logits: np.ndarray, k: int, expert_idx: np.ndarray, dy: np.ndarray,
                   yp_rows: np.ndarray, renorm: bool = False) -> np.ndarray:
    """Gradient of <dy, y> with respect to the logits, [T, E] float64, given
    the expert outputs yp_rows [T*k, d] (assignment order) the forward
    combined; the selection is held fixed."""
    logits = _f32(logits)
    T, E = logits.shape
    dy = _f32(dy)
    yp_rows = np.ascontiguousarray(yp_rows, np.float64)
    d = dy.shape[1]
    if dy.shape != (T, d) or yp_rows.shape != (T * k, d):
        raise ValueError("inconsistent shapes")
    ei = np.ascontiguousarray(expert_idx, np.int32)
    out = np.zeros((T, E), np.float64)
    rc = lib().orc_route_backward(_p(logits, _f32p), T, E, k, int(bool(renorm)), _p(ei, _i32p),
                                  _p(dy, _f32p), _p(yp_rows, _f64p), d, _p(out, _f64p))
    if rc != 0:
        raise ValueError("orc_route_backward rejected its arguments")
    return out


def permute_pad(x: np.ndarray, k: int, dest_row: np.ndarray, Tp: int, scale=None,
                prec: str = "bf16") -> np.ndarray:
    """Expert-grouped, zero-padded copy of x: [Tp, d] float64."""
    x = _f32(x)
    T, d = x.shape
    dest_row = np.ascontiguousarray(dest_row, np.int32)
    xp = np.zeros((Tp, d), np.float64)
    sc = _f32(scale)
    rc = lib().orc_permute_pad(_p(x, _f32p), T, d, k, _p(dest_row, _i32p), _p(sc, _f32p),
                               PREC[prec], Tp, _p(xp, _f64p))
    if rc != 0:
        raise ValueError("orc_permute_pad rejected its arguments")
    return xp


def topology(bin_offsets: np.ndarray, E: int, F: int, block_rows: int = 128) -> dict:
    """Hybrid BCSR-COO topology and transpose index of the block-diagonal
    first-layer output, in blocks of block_rows x 128."""
    bo = np.ascontiguousarray(bin_offsets, np.int32)
    R = int(bo[E]) // block_rows
    cap = R * F
    row_ptr = np.zeros(R + 1, np.int32)
    col_idx = np.zeros(cap, np.int32)
    row_idx = np.zeros(cap, np.int32)
    col_ptr = np.zeros(E * F + 1, np.int32)
    trans_idx = np.zeros(cap, np.int32)
    nnz = lib().orc_topology(_p(bo, _i32p), E, F, block_rows, _p(row_ptr, _i32p),
                             _p(col_idx, _i32p),
                             _p(row_idx, _i32p), _p(col_ptr, _i32p), _p(trans_idx, _i32p))
    if nnz < 0:
        raise ValueError("orc_topology rejected its arguments")
    return {"nnz": int(nnz), "row_ptr": row_ptr, "col_idx": col_idx[:nnz],
            "row_idx": row_idx[:nnz], "col_ptr": col_ptr, "trans_idx": trans_idx[:nnz]}


class Layer:
    """Float oracle of one layer call.

    ``prec`` is the storage precision of A, the saved factors (what the
    backward keeps: GeLU'(h); SwiGLU silu(h) and u * silu'(h)), dYp, dH, y,
    dx and the weight gradients; ``prec_yp`` that of Yp and dXp ("f64"
    disables rounding)."""

    def __init__(self, x, W1, W2, expert_idx, gate, k, E, act="gelu", W3=None, dy=None,
                 prec="bf16", prec_yp=None):
        self.x = _f32(x)
        self.W1 = _f32(W1)
        self.W2 = _f32(W2)
        self.W3 = _f32(W3)
        self.dy = _f32(dy)
        self.expert_idx = np.ascontiguousarray(expert_idx, np.int32)
        self.gate = _f32(gate)
        T, d = self.x.shape
        Ef = self.W1.shape[1]
        if Ef % E or self.W2.shape != (Ef, d) or self.W1.shape[0] != d:
            raise ValueError("inconsistent layer shapes")
        self.T, self.d, self.k, self.E, self.f = T, d, k, E, Ef // E
        s = self._s = _Layer()
        s.T, s.d, s.E, s.f, s.k = T, d, E, Ef // E, k
        s.act = ACT[act]
        s.prec = PREC[prec]
        s.prec_yp = PREC[prec_yp or prec]
        s.x = _p(self.x, _f32p)
        s.W1 = _p(self.W1, _f32p)
        s.W3 = _p(self.W3, _f32p)
        s.W2 = _p(self.W2, _f32p)
        s.dy = _p(self.dy, _f32p)
        s.expert_idx = _p(self.expert_idx, _i32p)
        s.gate = _p(self.gate, _f32p)

    def _call(self, name, *args):
        rc = getattr(lib(), name)(C.byref(self._s), *args)
        if rc != 0:
            raise ValueError(f"{name} rejected its arguments")

    @property
    def swiglu(self):
        return self._s.act == ACT["swiglu"]

    def assign_forward(self, assigns):
        """Per assignment: the saved factors G, A = rd(act(h)), Yp.

        G is [n, f] = rd(GeLU'(h)) for GeLU; for SwiGLU it is [2, n, f]:
        G[0] = rd(silu(h)), G[1] = rd(u * silu'(h))."""
        a = np.ascontiguousarray(assigns, np.int64)
        n = len(a)
        G = np.zeros((2, n, self.f) if self.swiglu else (1, n, self.f))
        A = np.zeros((n, self.f))
        Yp = np.zeros((n, self.d))
        self._call("orc_assign_forward", _p(a, _i64p), n, _p(G[0], _f64p),
                   _p(G[1], _f64p) if self.swiglu else None, _p(A, _f64p), _p(Yp, _f64p))
        return (G if self.swiglu else G[0]), A, Yp

    def forward_tokens(self, tokens):
        t = np.ascontiguousarray(tokens, np.int64)
        y = np.zeros((len(t), self.d))
        self._call("orc_forward_tokens", _p(t, _i64p), len(t), _p(y, _f64p))
        return y

    def assign_backward(self, assigns):
        """Per assignment: dYp, dH, dXp.  dH is [n, f] for GeLU; for SwiGLU it
        is [2, n, f]: dH[0] the gate projection's (pairs with W1), dH[1] the
        up projection's (pairs with W3)."""
        a = np.ascontiguousarray(assigns, np.int64)
        n = len(a)
        dYp = np.zeros((n, self.d))
        dH = np.zeros((2, n, self.f) if self.swiglu else (1, n, self.f))
        dXp = np.zeros((n, self.d))
        self._call("orc_assign_backward", _p(a, _i64p), n, _p(dYp, _f64p), _p(dH[0], _f64p),
                   _p(dH[1], _f64p) if self.swiglu else None, _p(dXp, _f64p))
        return dYp, (dH if self.swiglu else dH[0]), dXp

    def backward_tokens(self, tokens):
        t = np.ascontiguousarray(tokens, np.int64)
        dx = np.zeros((len(t), self.d))
        self._call("orc_backward_tokens", _p(t, _i64p), len(t), _p(dx, _f64p))
        return dx

    def dW2_block(self, rows, cols):
        r = np.ascontiguousarray(rows, np.int64)
        c = np.ascontiguousarray(cols, np.int64)
        out = np.zeros((len(r), len(c)))
        self._call("orc_dW2_block", _p(r, _i64p), len(r), _p(c, _i64p), len(c), _p(out, _f64p))
        return out

    def dW1_block(self, rows, cols):
        r = np.ascontiguousarray(rows, np.int64)
        c = np.ascontiguousarray(cols, np.int64)
        out = np.zeros((len(r), len(c)))
        self._call("orc_dW1_block", _p(r, _i64p), len(r), _p(c, _i64p), len(c), _p(out, _f64p))
        return out

    def dW3_block(self, rows, cols):
        """Gradient of W3 (SwiGLU's up projection) at (rows = model dims,
        cols = hidden units)."""
        r = np.ascontiguousarray(rows, np.int64)
        c = np.ascontiguousarray(cols, np.int64)
        out = np.zeros((len(r), len(c)))
        self._call("orc_dW3_block", _p(r, _i64p), len(r), _p(c, _i64p), len(c), _p(out, _f64p))
        return out


def make_layer(x, W1, W2, route_out, k, E, act="gelu", W3=None, dy=None, prec="bf16",
               prec_yp=None) -> Layer:
    """Convenience: a :class:`Layer` over the oracle's own routing."""
    return Layer(x, W1, W2, route_out["expert_idx"], route_out["gate"], k, E, act=act, W3=W3,
                 dy=dy, prec=prec, prec_yp=prec_yp)


# ------------------------------------------------------------ block products
#
# The three products on given operands for the MoE topology the bins define
# (orc_sdd, orc_dsd, orc_dstd in oracle.c: section 1.2's SDD and DSD, section
# 1.3's DSTD through the transpose index).  Dense operands are 2-D fp32 arrays
# of the stored values; block arrays are [planes * nnz, 128, 128] or flat.

SDD_EPI = {"none": 0, "gelu": 1, "silu_mul": 2, "gelu_bwd": 3, "silu_mul_bwd": 4}


def _nnz(bin_offsets, E, F, br):
    return int(bin_offsets[E]) // br * F


def sdd(a, b, K, bin_offsets, E, F, epilogue="none", prec="bf16", b2=None, trans_b=False,
        aux_in=None, want_aux=False, block_rows=128):
    """Blocks [planes * nnz, block_rows, 128] of the first-layer product (and
    the saved factors when want_aux, for gelu / silu_mul)."""
    a, b, b2 = _f32(a), _f32(b), _f32(b2)
    bo = np.ascontiguousarray(bin_offsets, np.int32)
    br = int(block_rows)
    nnz = _nnz(bo, E, F, br)
    epi = SDD_EPI[epilogue]
    planes = 2 if epi == 4 else 1
    out = np.zeros((planes * nnz, br, 128))
    aux = np.zeros(((2 if epi == 2 else 1) * nnz, br, 128)) if want_aux else None
    ai = None if aux_in is None else _f32(aux_in).reshape(-1)
    if b2 is not None and b2.shape != b.shape:
        raise ValueError("b2 must have b's shape")
    rc = lib().orc_sdd(_p(a, _f32p), a.shape[1], _p(b, _f32p), _p(b2, _f32p), b.shape[1],
                       int(bool(trans_b)), int(K), _p(bo, _i32p), E, F, br, epi, _p(ai, _f32p),
                       PREC[prec], _p(out, _f64p), _p(aux, _f64p))
    if rc != nnz:
        raise ValueError("orc_sdd rejected its arguments")
    return (out, aux) if want_aux else out


def dsd(blocks, bin_offsets, E, F, b, N, prec="bf16", trans_b=False, blocks2=None, b2=None,
        block_rows=128):
    """Rows [Tp, N] of the sparse x dense product (two block sets summed
    when blocks2 / b2 are given)."""
    bl, bl2 = _f32(blocks).reshape(-1), None if blocks2 is None else _f32(blocks2).reshape(-1)
    b, b2 = _f32(b), _f32(b2)
    bo = np.ascontiguousarray(bin_offsets, np.int32)
    Tp = int(bo[E])
    c = np.zeros((Tp, N))
    rc = lib().orc_dsd(_p(bl, _f32p), _p(bl2, _f32p), _p(bo, _i32p), E, F, int(block_rows),
                       _p(b, _f32p), _p(b2, _f32p), b.shape[1], int(bool(trans_b)), int(N),
                       PREC[prec], _p(c, _f64p))
    if rc != Tp:
        raise ValueError("orc_dsd rejected its arguments")
    return c


def dstd(blocks, bin_offsets, E, F, dmat, N, prec="bf16", block_rows=128):
    """The weight-gradient product [E * F * 128, N] (untransposed)."""
    bl, dm = _f32(blocks).reshape(-1), _f32(dmat)
    bo = np.ascontiguousarray(bin_offsets, np.int32)
    C_ = np.zeros((E * F * 128, N))
    rc = lib().orc_dstd(_p(bl, _f32p), _p(bo, _i32p), E, F, int(block_rows), _p(dm, _f32p),
                        dm.shape[1], int(N), PREC[prec], _p(C_, _f64p))
    if rc != 0:
        raise ValueError("orc_dstd rejected its arguments")
    return C_
