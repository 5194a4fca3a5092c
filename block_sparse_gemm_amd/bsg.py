"""Thin ctypes binding of ``include/bsg.h`` (libbsg.so).

Each function has the name of its C entry point without the ``bsg_``
prefix and only marshals arguments: torch tensors in, raw device pointers,
sizes and the current HIP stream out.  Every step of the layer runs in the
library's gfx950 kernels; there is no fallback of any kind: if the library
is missing this module raises on first use.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libbsg.so")

OK, EINVAL, EUNSUPPORTED, EHIP = 0, -1, -2, -3
F32, BF16 = 0, 1
EPI_NONE, EPI_GELU, EPI_SILU_MUL, EPI_GELU_BWD, EPI_SILU_MUL_BWD = 0, 1, 2, 3, 4
BLOCK = 128
MAX_EXPERTS = 1024
MAX_TOPK = 32
ROUTE_SCRATCH_BYTES = 4 << 20   # BSG_ROUTE_SCRATCH_BYTES

EPILOGUES = {"none": EPI_NONE, "gelu": EPI_GELU, "silu_mul": EPI_SILU_MUL,
             "gelu_bwd": EPI_GELU_BWD, "silu_mul_bwd": EPI_SILU_MUL_BWD}

# Every symbol include/bsg.h declares.
SYMBOLS = ("bsg_max_padded_rows", "bsg_topology_sizes", "bsg_route_workspace_bytes", "bsg_route",
           "bsg_route_noalloc",
           "bsg_route_backward", "bsg_permute_pad", "bsg_permute_pad_gate_backward",
           "bsg_build_topology", "bsg_route_topology", "bsg_route_permute_topology", "bsg_sdd", "bsg_dsd", "bsg_dsd_workspace_bytes",
           "bsg_dsd_combine_top1", "bsg_dstd",
           "bsg_unpermute_combine", "bsg_stream_copy", "bsg_status_string", "bsg_last_error")


class BsgError(RuntimeError):
    def __init__(self, call, status, detail):
        super().__init__(f"{call}: status {status} ({detail})")
        self.status = status


class TopoSizes(C.Structure):
    _fields_ = [("row_blocks_max", C.c_int64), ("nnz_max", C.c_int64), ("n_cols", C.c_int64),
                ("row_tiles_max", C.c_int64)]


class TopologyStruct(C.Structure):
    _fields_ = [("row_ptr", C.c_void_p), ("col_idx", C.c_void_p), ("row_idx", C.c_void_p),
                ("col_ptr", C.c_void_p), ("trans_idx", C.c_void_p), ("row_tiles", C.c_void_p),
                ("expert_order", C.c_void_p), ("meta", C.c_void_p),
                ("E", C.c_int32), ("F", C.c_int32), ("block_rows", C.c_int32),
                ("Tp_max", C.c_int64)]


_lib = None


def lib():
    """Load libbsg.so (built by ``python -m block_sparse_gemm_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run python -m block_sparse_gemm_amd.build")
        L = C.CDLL(LIB_PATH)
        vp, i64, i32, sz = C.c_void_p, C.c_int64, C.c_int, C.c_size_t
        L.bsg_max_padded_rows.restype = i64
        L.bsg_max_padded_rows.argtypes = [i64, i32, i32, i32]
        L.bsg_topology_sizes.restype = i32
        L.bsg_topology_sizes.argtypes = [i64, i32, i32, i32, C.POINTER(TopoSizes)]
        L.bsg_route_workspace_bytes.restype = sz
        L.bsg_route_workspace_bytes.argtypes = [i64, i32, i32]
        L.bsg_route.restype = i32
        L.bsg_route.argtypes = [vp, i64, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, sz, vp]
        L.bsg_stream_copy.restype = i32
        L.bsg_stream_copy.argtypes = [vp, vp, sz, vp]
        L.bsg_route_noalloc.restype = i32
        L.bsg_route_noalloc.argtypes = [vp, i64, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp]
        L.bsg_route_backward.restype = i32
        L.bsg_route_backward.argtypes = [vp, i64, i32, i32, i32, vp, vp, vp, i32, i32, vp, i32,
                                         i64, vp, vp]
        L.bsg_permute_pad.restype = i32
        L.bsg_permute_pad.argtypes = [vp, i32, i64, i32, i32, vp, vp, vp, vp, i32, i32, i64, vp, vp,
                                      vp]
        L.bsg_permute_pad_gate_backward.restype = i32
        L.bsg_permute_pad_gate_backward.argtypes = [vp, i32, i64, i32, i32, vp, vp, vp, vp, i32,
                                                    i32, i64, vp, vp, vp, i32, vp, vp, i32, i64,
                                                    vp, vp]
        L.bsg_build_topology.restype = i32
        L.bsg_build_topology.argtypes = [vp, i32, i32, i64, C.POINTER(TopologyStruct), vp]
        L.bsg_route_topology.restype = i32
        L.bsg_route_topology.argtypes = [vp, i64, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, sz,
                                         i32, i64, C.POINTER(TopologyStruct), vp]
        L.bsg_route_permute_topology.restype = i32
        L.bsg_route_permute_topology.argtypes = [vp, i64, i32, i32, i32, i32, vp, vp, vp, vp, vp,
                                                 vp, sz, vp, i32, i32, i64, vp, vp, i32,
                                                 C.POINTER(TopologyStruct), vp]
        L.bsg_sdd.restype = i32
        L.bsg_sdd.argtypes = [vp, i64, vp, vp, i64, i32, i32, C.POINTER(TopologyStruct), i32, vp,
                              vp, vp, i32, vp]
        L.bsg_dsd.restype = i32
        L.bsg_dsd.argtypes = [vp, vp, C.POINTER(TopologyStruct), vp, vp, i64, i32, i32, vp, i64,
                              i32, i32, vp, sz, vp]
        L.bsg_dsd_workspace_bytes.restype = i32
        L.bsg_dsd_workspace_bytes.argtypes = [vp, C.POINTER(i64)]
        L.bsg_dsd_combine_top1.restype = i32
        L.bsg_dsd_combine_top1.argtypes = [vp, C.POINTER(TopologyStruct), vp, i64, i32, i32, vp,
                                           i64, vp, vp, vp, i64, i32, vp]
        L.bsg_dstd.restype = i32
        L.bsg_dstd.argtypes = [vp, C.POINTER(TopologyStruct), vp, i64, i32, vp, i64, i32, i32,
                               vp]
        L.bsg_unpermute_combine.restype = i32
        L.bsg_unpermute_combine.argtypes = [vp, i32, i64, vp, vp, i64, i32, i32, vp, i32, vp]
        L.bsg_status_string.restype = C.c_char_p
        L.bsg_status_string.argtypes = [i32]
        L.bsg_last_error.restype = C.c_char_p
        L.bsg_last_error.argtypes = []
        _lib = L
    return _lib


def _check(call: str, status: int) -> None:
    if status != OK:
        raise BsgError(call, status, lib().bsg_last_error().decode())


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream():
    if torch.cuda.is_available():
        return C.c_void_p(torch.cuda.current_stream().cuda_stream)
    return None


def dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def torch_dtype(code: int):
    return torch.bfloat16 if code == BF16 else torch.float32


def _ld(t: torch.Tensor) -> int:
    assert t.dim() == 2 and t.stride(1) == 1, "operands must be row-major 2-D views"
    return t.stride(0)


# ------------------------------------------------------------- size queries

def max_padded_rows(T: int, k: int, E: int, bin_rows: int = BLOCK) -> int:
    return int(lib().bsg_max_padded_rows(T, k, E, bin_rows))


def topology_sizes(Tp_max: int, E: int, f: int, block_rows: int = BLOCK) -> TopoSizes:
    out = TopoSizes()
    _check("topology_sizes", lib().bsg_topology_sizes(Tp_max, E, f, block_rows, C.byref(out)))
    return out


def route_workspace_bytes(T: int, k: int, E: int) -> int:
    return int(lib().bsg_route_workspace_bytes(T, k, E))


# ------------------------------------------------------------------ topology

class Topology:
    """Device buffers of one hybrid BCSR-COO topology (capacity for Tp_max),
    in blocks of block_rows (128, or 64 for bins of 64 rows) x 128."""

    def __init__(self, Tp_max: int, E: int, f: int, device="cuda", block_rows: int = BLOCK):
        sz = topology_sizes(Tp_max, E, f, block_rows)
        i32 = dict(dtype=torch.int32, device=device)
        self.E, self.F, self.f, self.Tp_max = E, f // BLOCK, f, Tp_max
        self.block_rows = block_rows
        self.row_blocks_max, self.nnz_max = int(sz.row_blocks_max), int(sz.nnz_max)
        self.row_ptr = torch.zeros(self.row_blocks_max + 1, **i32)
        self.col_idx = torch.zeros(self.nnz_max, **i32)
        self.row_idx = torch.zeros(self.nnz_max, **i32)
        self.col_ptr = torch.zeros(E * self.F + 1, **i32)
        self.trans_idx = torch.zeros(self.nnz_max, **i32)
        self.row_tiles_max = int(sz.row_tiles_max)
        self.row_tiles = torch.zeros(self.row_tiles_max, **i32)
        self.expert_order = torch.zeros(E, **i32)
        self.meta = torch.zeros(4, **i32)
        self.struct = TopologyStruct(self.row_ptr.data_ptr(), self.col_idx.data_ptr(),
                                     self.row_idx.data_ptr(), self.col_ptr.data_ptr(),
                                     self.trans_idx.data_ptr(), self.row_tiles.data_ptr(),
                                     self.expert_order.data_ptr(), self.meta.data_ptr(), E,
                                     self.F, block_rows, Tp_max)


# ------------------------------------------------------------------- calls

def route(logits, k, renorm, expert_idx, gate, dest_row, counts, bin_offsets, workspace,
          bin_rows=BLOCK):
    T, E = logits.shape
    _check("route", lib().bsg_route(_ptr(logits), T, E, k, int(bool(renorm)), bin_rows,
                                    _ptr(expert_idx),
                                    _ptr(gate), _ptr(dest_row), _ptr(counts), _ptr(bin_offsets),
                                    _ptr(workspace), workspace.numel() * workspace.element_size(),
                                    _stream()))


def route_noalloc(logits, k, renorm, expert_idx, gate, dest_row, counts, bin_offsets,
                  bin_rows=BLOCK):
    T, E = logits.shape
    _check("route_noalloc", lib().bsg_route_noalloc(
        _ptr(logits), T, E, k, int(bool(renorm)), bin_rows, _ptr(expert_idx), _ptr(gate),
        _ptr(dest_row), _ptr(counts), _ptr(bin_offsets), _stream()))


def route_backward(logits, k, renorm, expert_idx, dest_row, dy, yp, dlogits):
    T, E = logits.shape
    _check("route_backward", lib().bsg_route_backward(
        _ptr(logits), T, E, k, int(bool(renorm)), _ptr(expert_idx), _ptr(dest_row), _ptr(dy),
        dtype_code(dy), dy.shape[1], _ptr(yp), dtype_code(yp), _ld(yp), _ptr(dlogits),
        _stream()))


def permute_pad(x, k, dest_row, scale, counts, bin_offsets, E, Tp_max, row_src, xp,
                bin_rows=BLOCK):
    T, d = x.shape
    _check("permute_pad", lib().bsg_permute_pad(_ptr(x), dtype_code(x), T, d, k, _ptr(dest_row),
                                                _ptr(scale), _ptr(counts), _ptr(bin_offsets), E,
                                                bin_rows, Tp_max, _ptr(row_src), _ptr(xp),
                                                _stream()))


def permute_pad_gate_backward(dy, k, dest_row, gate, counts, bin_offsets, E, Tp_max, row_src,
                              dyp, logits, renorm, expert_idx, yp, dlogits, bin_rows=BLOCK):
    T, d = dy.shape
    _check("permute_pad_gate_backward", lib().bsg_permute_pad_gate_backward(
        _ptr(dy), dtype_code(dy), T, d, k, _ptr(dest_row), _ptr(gate), _ptr(counts),
        _ptr(bin_offsets), E, bin_rows, Tp_max, _ptr(row_src), _ptr(dyp), _ptr(logits),
        int(bool(renorm)), _ptr(expert_idx), _ptr(yp), dtype_code(yp), _ld(yp), _ptr(dlogits),
        _stream()))


def build_topology(bin_offsets, E, f, Tp_max, topo: Topology):
    _check("build_topology", lib().bsg_build_topology(_ptr(bin_offsets), E, f, Tp_max,
                                                      C.byref(topo.struct), _stream()))


def route_topology(logits, k, renorm, expert_idx, gate, dest_row, counts, bin_offsets, workspace,
                   f, Tp_max, topo: Topology, bin_rows=BLOCK):
    """route + build_topology, the topology written by the routing's own launch."""
    T, E = logits.shape
    _check("route_topology", lib().bsg_route_topology(
        _ptr(logits), T, E, k, int(bool(renorm)), bin_rows, _ptr(expert_idx), _ptr(gate),
        _ptr(dest_row), _ptr(counts), _ptr(bin_offsets), _ptr(workspace),
        workspace.numel() * workspace.element_size(), f, Tp_max, C.byref(topo.struct),
        _stream()))


def route_permute_topology(logits, k, renorm, expert_idx, gate, dest_row, counts, bin_offsets,
                           workspace, x, Tp_max, row_src, xp, f=0, topo: Topology = None,
                           bin_rows=BLOCK):
    """route + permute_pad (no scale) + build_topology (topo may be None) in
    the routing's two launches."""
    T, E = logits.shape
    _check("route_permute_topology", lib().bsg_route_permute_topology(
        _ptr(logits), T, E, k, int(bool(renorm)), bin_rows, _ptr(expert_idx), _ptr(gate),
        _ptr(dest_row), _ptr(counts), _ptr(bin_offsets), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _ptr(x), dtype_code(x), x.shape[1],
        Tp_max, _ptr(row_src), _ptr(xp), f, C.byref(topo.struct) if topo is not None else None,
        _stream()))


def sdd(a, b, K, topo: Topology, epilogue, out_blocks, b2=None, trans_b=False, aux_in=None,
        aux_out=None):
    epi = EPILOGUES[epilogue] if isinstance(epilogue, str) else int(epilogue)
    _check("sdd", lib().bsg_sdd(_ptr(a), _ld(a), _ptr(b), _ptr(b2), _ld(b), int(bool(trans_b)),
                                K, C.byref(topo.struct), epi, _ptr(aux_in), _ptr(out_blocks),
                                _ptr(aux_out), dtype_code(a), _stream()))


def dsd(blocks, topo: Topology, b, N, c, trans_b=False, blocks2=None, b2=None, workspace=None):
    """bsg_dsd; workspace (a device tensor, or None) lets the product split
    its last round (see dsd_workspace_bytes)."""
    nbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check("dsd", lib().bsg_dsd(_ptr(blocks), _ptr(blocks2), C.byref(topo.struct), _ptr(b),
                                _ptr(b2), _ld(b), int(bool(trans_b)), N, _ptr(c), _ld(c),
                                dtype_code(c), dtype_code(blocks), _ptr(workspace), nbytes,
                                _stream()))


def dsd_workspace_bytes() -> int:
    """Bytes of a bsg_dsd workspace that allows every split of its last round
    on the current device (one 256 KiB share per compute unit)."""
    out = C.c_int64(0)
    _check("dsd_workspace_bytes", lib().bsg_dsd_workspace_bytes(_stream(), C.byref(out)))
    return int(out.value)


def dsd_combine_top1(blocks, topo: Topology, b, N, c, row_src, gate, y, trans_b=False):
    """bsg_dsd + bsg_unpermute_combine for top-1 routing in one launch (c may
    be None: only y is written)."""
    _check("dsd_combine_top1", lib().bsg_dsd_combine_top1(
        _ptr(blocks), C.byref(topo.struct), _ptr(b), _ld(b), int(bool(trans_b)), N, _ptr(c),
        _ld(c) if c is not None else 0, _ptr(row_src), _ptr(gate), _ptr(y), _ld(y),
        dtype_code(blocks), _stream()))


def dstd(blocks, topo: Topology, dmat, N, c, trans_c=False):
    _check("dstd", lib().bsg_dstd(_ptr(blocks), C.byref(topo.struct), _ptr(dmat), _ld(dmat), N,
                                  _ptr(c), _ld(c), int(bool(trans_c)), dtype_code(blocks),
                                  _stream()))


def unpermute_combine(yp, dest_row, gate, T, k, d, y):
    _check("unpermute_combine", lib().bsg_unpermute_combine(
        _ptr(yp), dtype_code(yp), _ld(yp), _ptr(dest_row), _ptr(gate), T, k, d, _ptr(y),
        dtype_code(y), _stream()))


def stream_copy(src, dst, nbytes=None):
    """Copy nbytes (default: all of src) from src to dst with the library's
    streaming copy (a measurement ceiling, not a step of the layer)."""
    n = src.numel() * src.element_size() if nbytes is None else int(nbytes)
    _check("stream_copy", lib().bsg_stream_copy(_ptr(src), _ptr(dst), n, _stream()))
