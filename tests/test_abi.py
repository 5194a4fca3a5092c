"""The C ABI without a GPU: the library loads, exports every symbol the
header declares, answers the size queries with their closed forms, and
rejects bad arguments before any HIP call."""
import ctypes as C
import os
import re

import pytest

from block_sparse_gemm_amd import bsg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bsg.h")

P = C.c_void_p(0x10000)       # a fake, aligned, non-null pointer: never dereferenced
MIS = C.c_void_p(0x10004)     # 4-byte but not 16-byte aligned


@pytest.fixture(scope="module")
def L():
    return bsg.lib()


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(bsg_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(L):
    syms = declared_symbols()
    assert len(syms) >= 12
    for s in syms:
        assert hasattr(L, s), s
    assert set(bsg.SYMBOLS) == set(syms)


def test_size_queries(L):
    for T, k, E in [(1, 1, 1), (256, 1, 4), (16384, 1, 64), (32768, 1, 64), (8192, 2, 8),
                    (65536, 2, 64), (3, 2, 64)]:
        A = T * k
        want = (A + 127 * min(E, A)) // 128 * 128
        assert bsg.max_padded_rows(T, k, E) == want
        want = (A + 255 * min(E, A)) // 256 * 256
        assert bsg.max_padded_rows(T, k, E, 256) == want
        want = (A + 63 * min(E, A)) // 64 * 64
        assert bsg.max_padded_rows(T, k, E, 64) == want
    assert bsg.max_padded_rows(0, 1, 1) == -1
    assert bsg.max_padded_rows(4, 3, 2) == -1
    assert bsg.max_padded_rows(4, 1, 2, 32) == -1
    assert bsg.max_padded_rows(4, 1, 2, 200) == -1
    s = bsg.topology_sizes(139136, 64, 4096)
    assert (s.row_blocks_max, s.nnz_max, s.n_cols) == (1087, 1087 * 32, 64 * 32)
    assert s.row_tiles_max == (1087 + 64 + 1) // 2
    # blocks of 64 rows: tiles of four block rows
    s = bsg.topology_sizes(139136, 64, 4096, 64)
    assert (s.row_blocks_max, s.nnz_max) == (2174, 2174 * 32)
    assert s.row_tiles_max == (2174 + 3 * (64 + 1)) // 4
    with pytest.raises(bsg.BsgError):
        bsg.topology_sizes(1280, 4, 256, 32)
    assert bsg.route_workspace_bytes(65536, 2, 64) == 1024 * 64 * 4
    assert bsg.route_workspace_bytes(65, 1, 3) == 2 * 3 * 4
    assert bsg.route_workspace_bytes(10, 3, 2) == 0
    with pytest.raises(bsg.BsgError):
        bsg.topology_sizes(100, 4, 256)
    with pytest.raises(bsg.BsgError):
        bsg.topology_sizes(1280, 4, 200)


def _err(L):
    return L.bsg_last_error().decode()


def test_route_validation(L):
    ws = 1 << 20
    ok_args = [P, 100, 8, 2, 0, 128, P, P, P, P, P, P, ws, None]

    def call(**over):
        a = list(ok_args)
        names = ["logits", "T", "E", "k", "renorm", "bin", "expert_idx", "gate", "dest_row",
                 "counts", "bin_offsets", "ws", "wsb", "stream"]
        for key, v in over.items():
            a[names.index(key)] = v
        return L.bsg_route(*a)

    assert call(logits=None) == bsg.EINVAL
    assert call(T=0) == bsg.EINVAL
    assert call(E=0) == bsg.EINVAL
    assert call(E=2000) == bsg.EINVAL
    assert call(k=9) == bsg.EINVAL
    assert call(k=0) == bsg.EINVAL
    assert call(E=64, k=40) == bsg.EUNSUPPORTED
    assert call(gate=None) == bsg.EINVAL
    assert call(ws=None) == bsg.EINVAL
    assert call(wsb=4) == bsg.EINVAL and "workspace" in _err(L)
    assert call(counts=C.c_void_p(0x10002)) == bsg.EINVAL
    assert call(bin=32) == bsg.EINVAL
    assert call(bin=100) == bsg.EINVAL


def test_route_backward_validation(L):
    ok = [P, 100, 8, 2, 0, P, P, P, bsg.BF16, 128, P, bsg.BF16, 128, P, None]
    names = ["logits", "T", "E", "k", "renorm", "expert_idx", "dest_row", "dy", "dyt", "d", "yp",
             "ypt", "ld", "dlogits", "stream"]

    def call(**over):
        a = list(ok)
        for key, v in over.items():
            a[names.index(key)] = v
        return L.bsg_route_backward(*a)

    assert call(logits=None) == bsg.EINVAL
    assert call(T=0) == bsg.EINVAL
    assert call(k=9) == bsg.EINVAL
    assert call(E=64, k=40) == bsg.EUNSUPPORTED
    assert call(d=100) == bsg.EINVAL
    assert call(ld=64) == bsg.EINVAL
    assert call(dyt=7) == bsg.EINVAL
    assert call(yp=MIS) == bsg.EINVAL
    assert call(dlogits=None) == bsg.EINVAL


def test_permute_pad_validation(L):
    T, d, k, E = 100, 128, 2, 8
    Tp = bsg.max_padded_rows(T, k, E)
    base = [P, bsg.BF16, T, d, k, P, None, P, P, E, 128, Tp, P, P, None]
    assert L.bsg_permute_pad(*[None if i == 0 else v for i, v in enumerate(base)]) == bsg.EINVAL
    b = list(base); b[1] = 7
    assert L.bsg_permute_pad(*b) == bsg.EINVAL
    b = list(base); b[3] = 100  # 200 bytes per row: not 16-byte aligned rows
    assert L.bsg_permute_pad(*b) == bsg.EINVAL
    b = list(base); b[11] = Tp - 128
    assert L.bsg_permute_pad(*b) == bsg.EINVAL and "Tp_max" in _err(L)
    b = list(base); b[10] = 256  # the 256-row bins need a larger Tp_max
    assert L.bsg_permute_pad(*b) == bsg.EINVAL and "Tp_max" in _err(L)
    b = list(base); b[10] = 32
    assert L.bsg_permute_pad(*b) == bsg.EINVAL
    b = list(base); b[13] = MIS
    assert L.bsg_permute_pad(*b) == bsg.EINVAL
    b = list(base); b[4] = 9
    assert L.bsg_permute_pad(*b) == bsg.EINVAL


def test_permute_pad_gate_backward_validation(L):
    T, d, k, E = 100, 128, 2, 8
    Tp = bsg.max_padded_rows(T, k, E)
    names = ["dy", "dt", "T", "d", "k", "dest", "gate", "counts", "bo", "E", "bin", "Tp", "rs",
             "dyp", "logits", "renorm", "ei", "yp", "ypt", "ld", "dl", "stream"]
    ok = [P, bsg.BF16, T, d, k, P, P, P, P, E, 128, Tp, P, P, P, 0, P, P, bsg.BF16, d, P, None]

    def call(**over):
        a = list(ok)
        for key, v in over.items():
            a[names.index(key)] = v
        return L.bsg_permute_pad_gate_backward(*a)

    assert call(dy=None) == bsg.EINVAL
    assert call(gate=None) == bsg.EINVAL
    assert call(dl=None) == bsg.EINVAL
    assert call(yp=MIS) == bsg.EINVAL
    assert call(Tp=Tp - 128) == bsg.EINVAL and "Tp_max" in _err(L)
    assert call(ld=64) == bsg.EINVAL
    assert call(d=100) == bsg.EINVAL
    assert call(dt=bsg.F32, ypt=bsg.BF16) == bsg.EUNSUPPORTED
    assert call(bin=32) == bsg.EINVAL
    assert call(E=64, k=40) == bsg.EUNSUPPORTED


def test_dsd_combine_top1_validation(L):
    t = fake_topo(E=4, f=256)
    names = ["blocks", "topo", "b", "ldb", "tb", "N", "c", "ldc", "rs", "gate", "y", "ldy", "dt",
             "stream"]
    ok = [P, C.byref(t), P, 256, 0, 256, P, 256, P, None, P, 256, bsg.BF16, None]

    def call(**over):
        a = list(ok)
        for key, v in over.items():
            a[names.index(key)] = v
        return L.bsg_dsd_combine_top1(*a)

    assert call(blocks=None) == bsg.EINVAL
    assert call(y=None) == bsg.EINVAL
    assert call(rs=None) == bsg.EINVAL
    assert call(ldy=128) == bsg.EINVAL
    assert call(c=MIS) == bsg.EINVAL
    assert call(ldc=128) == bsg.EINVAL
    assert call(N=200) == bsg.EINVAL
    assert call(dt=bsg.F32) == bsg.EUNSUPPORTED
    assert call(gate=C.c_void_p(0x10002)) == bsg.EINVAL


def fake_topo(E=4, f=256, Tp=1024, **over):
    t = bsg.TopologyStruct(0x10000, 0x20000, 0x30000, 0x40000, 0x50000, 0x70000, 0x80000,
                           0x60000, E, f // 128, 128, Tp)
    for k, v in over.items():
        setattr(t, k, v)
    return t


def test_build_topology_validation(L):
    t = fake_topo()
    assert L.bsg_build_topology(None, 4, 256, 1024, C.byref(t), None) == bsg.EINVAL
    assert L.bsg_build_topology(P, 4, 256, 1024, None, None) == bsg.EINVAL
    assert L.bsg_build_topology(P, 4, 200, 1024, C.byref(t), None) == bsg.EINVAL
    assert L.bsg_build_topology(P, 5, 256, 1024, C.byref(t), None) == bsg.EINVAL
    assert "capacity" in _err(L)
    t2 = fake_topo(row_idx=None)
    assert L.bsg_build_topology(P, 4, 256, 1024, C.byref(t2), None) == bsg.EINVAL
    t4 = fake_topo(expert_order=None)
    assert L.bsg_build_topology(P, 4, 256, 1024, C.byref(t4), None) == bsg.EINVAL
    t3 = fake_topo(Tp=1000)
    assert L.bsg_build_topology(P, 4, 256, 1000, C.byref(t3), None) == bsg.EINVAL
    t5 = fake_topo(block_rows=96)
    assert L.bsg_build_topology(P, 4, 256, 1024, C.byref(t5), None) == bsg.EINVAL
    assert "block_rows" in _err(L)


def test_route_topology_validation(L):
    """Every argument rule of route and of build_topology, checked before any
    launch (the pointers are never dereferenced)."""
    t = fake_topo(E=8)
    ok = [P, 100, 8, 2, 0, 128, P, P, P, P, P, P, 1 << 20, 256, 1024, C.byref(t), None]
    names = ["logits", "T", "E", "k", "renorm", "bin", "expert_idx", "gate", "dest_row",
             "counts", "bin_offsets", "ws", "wsb", "f", "Tp", "topo", "stream"]

    def call(**over):
        a = list(ok)
        for key, v in over.items():
            a[names.index(key)] = v
        return L.bsg_route_topology(*a)

    assert call(logits=None) == bsg.EINVAL
    assert call(k=9) == bsg.EINVAL
    assert call(E=64, k=40) == bsg.EUNSUPPORTED
    assert call(wsb=4) == bsg.EINVAL and "workspace" in _err(L)
    assert call(bin=32) == bsg.EINVAL
    assert call(f=384) == bsg.EINVAL and "capacity" in _err(L)
    assert call(f=200) == bsg.EINVAL
    assert call(Tp=2048) == bsg.EINVAL
    assert call(topo=None) == bsg.EINVAL
    t2 = fake_topo(E=8, meta=None)
    assert call(topo=C.byref(t2)) == bsg.EINVAL


def test_route_permute_topology_validation(L):
    """The rules of route, permute_pad (without a scale) and build_topology,
    checked before any launch; the topology is optional."""
    Tp = bsg.max_padded_rows(100, 2, 8)
    t = fake_topo(E=8, Tp=Tp)
    ok = [P, 100, 8, 2, 0, 128, P, P, P, P, P, P, 1 << 20, P, bsg.BF16, 256, Tp, P, P, 256,
          C.byref(t), None]
    names = ["logits", "T", "E", "k", "renorm", "bin", "expert_idx", "gate", "dest_row",
             "counts", "bin_offsets", "ws", "wsb", "x", "dt", "d", "Tp", "row_src", "xp", "f",
             "topo", "stream"]

    def call(**over):
        a = list(ok)
        for key, v in over.items():
            a[names.index(key)] = v
        return L.bsg_route_permute_topology(*a)

    assert call(logits=None) == bsg.EINVAL
    assert call(wsb=4) == bsg.EINVAL and "workspace" in _err(L)
    assert call(x=C.c_void_p(0x10004)) == bsg.EINVAL
    assert call(xp=None) == bsg.EINVAL
    assert call(row_src=None) == bsg.EINVAL
    assert call(d=100) == bsg.EINVAL
    assert call(dt=7) == bsg.EINVAL
    assert call(Tp=256) == bsg.EINVAL and "padded-row bound" in _err(L)
    assert call(f=384) == bsg.EINVAL and "capacity" in _err(L)
    assert call(bin=32) == bsg.EINVAL


def test_sdd_validation(L):
    t = fake_topo(E=4, f=256)
    ncol = 4 * 256

    def call(a=P, lda=256, b=P, b2=None, ldb=ncol, trans_b=0, K=256, topo=t, epi=bsg.EPI_GELU,
             aux_in=None, out=P, aux_out=None, dtype=bsg.BF16):
        return L.bsg_sdd(a, lda, b, b2, ldb, trans_b, K, C.byref(topo) if topo else None, epi,
                         aux_in, out, aux_out, dtype, None)

    assert call(a=None) == bsg.EINVAL
    assert call(a=MIS) == bsg.EINVAL
    assert call(K=100) == bsg.EINVAL
    assert call(K=96) == bsg.EINVAL          # not a multiple of 64 for bf16
    assert call(lda=128) == bsg.EINVAL       # lda < K
    assert call(ldb=512) == bsg.EINVAL       # ldb < E*f for trans_b = 0
    assert call(trans_b=2) == bsg.EINVAL
    assert call(epi=9) == bsg.EINVAL
    assert call(dtype=5) == bsg.EINVAL
    assert call(topo=None) == bsg.EINVAL
    assert call(epi=bsg.EPI_SILU_MUL) == bsg.EINVAL               # b2 missing
    assert call(epi=bsg.EPI_SILU_MUL, b2=P, trans_b=1, ldb=256) == bsg.EUNSUPPORTED
    assert call(epi=bsg.EPI_GELU_BWD) == bsg.EINVAL               # aux_in missing
    assert call(epi=bsg.EPI_NONE, aux_in=P) == bsg.EINVAL
    assert call(epi=bsg.EPI_NONE, aux_out=P) == bsg.EINVAL
    assert call(epi=bsg.EPI_GELU, b2=P) == bsg.EINVAL
    assert call(epi=bsg.EPI_SILU_MUL_BWD) == bsg.EINVAL           # aux_in missing
    assert call(epi=bsg.EPI_SILU_MUL_BWD, aux_in=P, b2=P) == bsg.EINVAL
    assert call(epi=bsg.EPI_SILU_MUL_BWD, aux_in=P, aux_out=P) == bsg.EINVAL
    assert call(epi=bsg.EPI_SILU_MUL, b2=P, aux_out=MIS) == bsg.EINVAL
    assert call(epi=5) == bsg.EINVAL


def test_dsd_dstd_validation(L):
    t = fake_topo(E=4, f=256)
    ncol = 4 * 256

    def dsd(blocks=P, blocks2=None, b=P, b2=None, ldb=256, trans_b=0, N=256, c=P, ldc=256,
            c_dtype=bsg.BF16, dtype=bsg.BF16, ws=None, ws_bytes=0):
        return L.bsg_dsd(blocks, blocks2, C.byref(t), b, b2, ldb, trans_b, N, c, ldc, c_dtype,
                         dtype, ws, ws_bytes, None)

    # the split workspace: 256-byte aligned, two 256 KiB shares at least
    assert dsd(ws=MIS, ws_bytes=1 << 20) == bsg.EINVAL and "aligned" in _err(L)
    assert dsd(ws=P, ws_bytes=(1 << 18) + 4096) == bsg.EINVAL and "two tile shares" in _err(L)

    assert dsd(N=200) == bsg.EINVAL
    assert dsd(ldb=128) == bsg.EINVAL
    assert dsd(trans_b=1) == bsg.EINVAL          # ldb < E*f for B transposed
    assert dsd(ldc=128) == bsg.EINVAL
    assert dsd(dtype=bsg.F32) == bsg.EUNSUPPORTED
    assert dsd(blocks=None) == bsg.EINVAL
    assert dsd(blocks2=P) == bsg.EINVAL          # the second set needs its B
    assert dsd(b2=P) == bsg.EINVAL               # ... and its blocks
    assert dsd(blocks2=MIS, b2=P) == bsg.EINVAL
    assert L.bsg_dstd(P, C.byref(t), P, 256, 256, P, 256, 1, bsg.BF16, None) == bsg.EINVAL
    assert L.bsg_dstd(P, C.byref(t), P, 128, 256, P, 256, 0, bsg.BF16, None) == bsg.EINVAL
    assert L.bsg_dstd(P, C.byref(t), P, 256, 256, P, ncol, 2, bsg.BF16, None) == bsg.EINVAL
    assert L.bsg_dstd(P, C.byref(t), P, 256, 192, P, 256, 0, bsg.BF16, None) == bsg.EINVAL
    assert L.bsg_dstd(P, C.byref(t), None, 256, 256, P, 256, 0, bsg.BF16, None) == bsg.EINVAL


def test_combine_validation(L):
    assert L.bsg_unpermute_combine(P, bsg.BF16, 256, P, None, 10, 2, 100, P, bsg.BF16,
                                   None) == bsg.EINVAL
    assert L.bsg_unpermute_combine(P, bsg.BF16, 64, P, None, 10, 2, 128, P, bsg.BF16,
                                   None) == bsg.EINVAL
    assert L.bsg_unpermute_combine(None, bsg.BF16, 128, P, None, 10, 2, 128, P, bsg.BF16,
                                   None) == bsg.EINVAL
    assert L.bsg_unpermute_combine(P, 3, 128, P, None, 10, 2, 128, P, bsg.BF16,
                                   None) == bsg.EINVAL
    assert L.bsg_unpermute_combine(P, bsg.BF16, 128, P, None, 10, 40, 128, P, bsg.BF16,
                                   None) == bsg.EINVAL


def test_status_strings(L):
    assert L.bsg_status_string(0) == b"ok"
    assert L.bsg_status_string(-1) == b"invalid argument"
    assert L.bsg_status_string(-2) == b"unsupported combination"
    assert L.bsg_status_string(-3) == b"HIP runtime error"
    assert L.bsg_status_string(7) == b"unknown status"


def test_leading_dimensions_beyond_32bit_panel_offsets(L):
    """The products reach a panel's rows through 32-bit byte offsets: a
    leading dimension whose last panel row lies 4 GiB or more past the
    panel's origin is refused, not wrapped (bf16: row 127 of a K-contiguous
    panel, K-row 31 of a panel contiguous along M or N)."""
    t = fake_topo(E=4, f=256)
    kc = 16909320    # 127 * kc * 2 + 64 > 2^32 - 1 (the largest accepted is 16909312)
    km = 69273664    # 31 * km * 2 + 256 > 2^32 - 1 (the largest accepted is 69273656)
    assert 127 * (kc - 8) * 2 + 64 <= 2**32 - 1 < 127 * kc * 2 + 64
    assert 31 * (km - 8) * 2 + 256 <= 2**32 - 1 < 31 * km * 2 + 256

    def sdd(lda=256, ldb=1024, trans_b=0):
        return L.bsg_sdd(P, lda, P, None, ldb, trans_b, 256, C.byref(t), bsg.EPI_GELU, None, P,
                         None, bsg.BF16, None)

    assert sdd(lda=kc) == bsg.EUNSUPPORTED and "32-bit" in _err(L)
    assert sdd(ldb=km) == bsg.EUNSUPPORTED
    assert sdd(ldb=kc, trans_b=1) == bsg.EUNSUPPORTED

    def dsd(ldb, trans_b):
        return L.bsg_dsd(P, None, C.byref(t), P, None, ldb, trans_b, 256, P, 256, bsg.BF16,
                         bsg.BF16, None, 0, None)

    assert dsd(km, 0) == bsg.EUNSUPPORTED
    assert dsd(kc, 1) == bsg.EUNSUPPORTED
    assert L.bsg_dsd_combine_top1(P, C.byref(t), P, kc, 1, 256, P, 256, P, None, P, 256,
                                  bsg.BF16, None) == bsg.EUNSUPPORTED
    assert L.bsg_dstd(P, C.byref(t), P, km, 256, P, 256, 0, bsg.BF16, None) == bsg.EUNSUPPORTED


def test_route_noalloc_validation(L):
    """The allocation-free routing call validates like bsg_route, and refuses
    a request whose per-chunk counts exceed its static device array, all
    before any HIP call."""
    ok = [P, 100, 8, 2, 0, 128, P, P, P, P, P, None]
    names = ["logits", "T", "E", "k", "renorm", "bin", "expert_idx", "gate", "dest_row",
             "counts", "bin_offsets", "stream"]

    def call(**over):
        a = list(ok)
        for key, v in over.items():
            a[names.index(key)] = v
        return L.bsg_route_noalloc(*a)

    assert call(logits=None) == bsg.EINVAL
    assert call(gate=None) == bsg.EINVAL
    assert call(T=0) == bsg.EINVAL
    assert call(k=9) == bsg.EINVAL
    assert call(E=64, k=40) == bsg.EUNSUPPORTED
    assert call(bin=32) == bsg.EINVAL
    assert call(counts=C.c_void_p(0x10002)) == bsg.EINVAL
    # ceil(T / 64) * E * 4 bytes of counts: 1025 chunks x 1024 experts > 4 MiB
    assert bsg.route_workspace_bytes(64 * 1025, 1, 1024) > bsg.ROUTE_SCRATCH_BYTES
    assert call(T=64 * 1025, E=1024, k=1) == bsg.EUNSUPPORTED and "scratch" in _err(L)


def test_stream_copy_validation(L):
    Q = C.c_void_p(0x100000)
    assert L.bsg_stream_copy(None, P, 64, None) == bsg.EINVAL
    assert L.bsg_stream_copy(P, MIS, 64, None) == bsg.EINVAL
    assert L.bsg_stream_copy(P, Q, 40, None) == bsg.EINVAL        # not a multiple of 16
    assert L.bsg_stream_copy(P, C.c_void_p(0x10010), 64, None) == bsg.EINVAL  # overlap
    assert "overlap" in _err(L)
