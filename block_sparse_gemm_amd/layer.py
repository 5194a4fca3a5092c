"""The dropless-MoE expert layer as a chain of the library's calls.

Forward (George Lin's Blog, MegaBlocks/FlexMoE post, sections 1.2-1.4):
    route (+ permute_pad and build_topology, both done by the routing's
    placement launch) -> sdd (+ activation) -> dsd -> unpermute_combine
Backward (plain calculus on the same products, weight gradients through the
transpose index as section 1.3 describes):
    permute_pad(dy, scale = gate) + route_backward(dy, Yp) = dlogits (the
    gate's gradient, selection fixed) in one pass over dy
    -> sdd(dYp, W2^T, GeLU') -> dsd(dH, W1^T) -> unpermute_combine(gate = 1) ;
    dstd(A, dYp) = dW2 ; dstd(dH, Xp)^T = dW1
SwiGLU experts keep silu(g) and u * silu'(g) from the forward; their
backward product gives the gate and the up projection's gradients (two
planes of dH), the input gradient is one two-set dsd (dH_gate W1^T +
dH_up W3^T), and dW1, dW3 are one dstd each.
With ``overlap`` set (the default when the products are short) the weight
gradients run on a second stream, each as soon as its inputs exist (dW2 beside the backward SDD product, dW1 (and dW3)
beside the input-gradient product), so the tail of one product's grid and
the other's fill the GPU together.

torch only allocates device memory and provides the stream; every step runs
in libbsg.so.  All buffers are sized once for the worst-case routing
(``max_padded_rows``), so a layer call never synchronises the host.
"""
from __future__ import annotations

import dataclasses

import torch

from . import bsg


@dataclasses.dataclass
class Shape:
    T: int
    d: int
    E: int
    f: int
    k: int
    act: str = "gelu"          # "gelu" or "swiglu"
    dtype: str = "bf16"        # "bf16" or "f32"
    yp_dtype: str = "bf16"     # storage of Yp / dXp
    renorm: bool = False
    backward: bool = False
    bin_rows: int = 128        # expert bins padded to a multiple of this (64, 128 or 256)

    @classmethod
    def of(cls, cfg) -> "Shape":
        """The shape of a workload description (synth.LayerConfig or alike)."""
        return cls(cfg.T, cfg.d, cfg.E, cfg.f, cfg.k, cfg.act, cfg.dtype, cfg.yp, cfg.renorm,
                   cfg.backward, getattr(cfg, "bin_rows", 128))

    @property
    def tdtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    @property
    def yp_tdtype(self):
        return torch.bfloat16 if (self.yp_dtype == "bf16" and self.dtype == "bf16") \
            else torch.float32


class Layer:
    """Preallocated device buffers + the forward/backward call chains."""

    def __init__(self, s: Shape, device="cuda"):
        self.s = s
        # optional callable(name, phase) run on the call's stream before
        # (phase "begin") and after (phase "end") each library call
        self.mark = None
        # True: the weight gradients run on a second stream beside the
        # data-gradient chain.  Each product's grid covers every CU (one
        # workgroup per CU), so the second stream only fills grid tails.
        # That pays when the products are short (at most about 0.4 TFLOP
        # each, a few hundred microseconds, where the tails are a large
        # share): the MoE-Small-shaped step measured 1.52 -> 1.49 ms.  With
        # longer products (the skewed and Mixtral-shaped layers) it measured
        # no faster, so there every call stays in order on the caller's
        # stream.  Set it to choose the schedule.
        self.overlap = s.backward and 2.0 * s.T * s.k * s.d * s.f <= 4e11
        # top-1 bf16 layers: the combine runs in the DSD's epilogue (forward:
        # y, and Yp when a backward follows; backward with GeLU experts: dx
        # straight from the product, no dXp)
        self.fuse_top1 = s.k == 1 and s.dtype == "bf16" and s.yp_tdtype == torch.bfloat16
        dev = torch.device(device)
        # plain DSDs whose tiles walk at least 32 K-blocks (f >= 4096, or the
        # SwiGLU backward's two block sets) split their last, partly filled
        # round of tiles through this workspace (None: never)
        F = s.f // bsg.BLOCK
        long_k = F >= 32 or (s.act == "swiglu" and s.backward and 2 * F >= 32)
        self.dsd_ws = torch.empty(bsg.dsd_workspace_bytes() // 4, dtype=torch.float32,
                                  device=dev) if long_k and not self.fuse_top1 else None
        i32 = dict(dtype=torch.int32, device=dev)
        A = s.T * s.k
        self.Tp_max = bsg.max_padded_rows(s.T, s.k, s.E, s.bin_rows)
        # bins of 64 rows need blocks of 64 rows (a block holds one expert's rows)
        self.block_rows = 64 if s.bin_rows == 64 else bsg.BLOCK
        self.topo = bsg.Topology(self.Tp_max, s.E, s.f, device=dev, block_rows=self.block_rows)
        nnz_max = self.topo.nnz_max
        br = self.block_rows
        dt, ydt = s.tdtype, s.yp_tdtype
        self.expert_idx = torch.zeros(A, **i32)
        self.gate = torch.zeros(A, dtype=torch.float32, device=dev)
        self.dest_row = torch.zeros(A, **i32)
        self.counts = torch.zeros(s.E, **i32)
        self.bin_offsets = torch.zeros(s.E + 1, **i32)
        self.route_ws = torch.zeros(max(1, bsg.route_workspace_bytes(s.T, s.k, s.E)),
                                    dtype=torch.uint8, device=dev)
        self.row_src = torch.zeros(self.Tp_max, **i32)
        self.xp = torch.zeros(self.Tp_max, s.d, dtype=dt, device=dev)
        self.act = torch.zeros(nnz_max * br, bsg.BLOCK, dtype=dt, device=dev)
        # what the backward keeps of the forward, block-major like A: GeLU'(h),
        # or for SwiGLU two planes, silu(g) then u * silu'(g)
        planes = 2 if s.act == "swiglu" else 1
        self.gp = torch.zeros(planes * nnz_max * br, bsg.BLOCK, dtype=dt, device=dev) \
            if s.backward else None
        self.yp = torch.zeros(self.Tp_max, s.d, dtype=ydt, device=dev)
        self.y = torch.zeros(s.T, s.d, dtype=dt, device=dev)
        if s.backward:
            self.dyp = torch.zeros(self.Tp_max, s.d, dtype=dt, device=dev)
            self.row_src_b = torch.zeros(self.Tp_max, **i32)
            # SwiGLU: plane 0 the gate projection's gradient, plane 1 the up's
            self.dh = torch.zeros_like(self.gp)
            self.dxp = torch.zeros(self.Tp_max, s.d, dtype=ydt, device=dev)
            self.dx = torch.zeros(s.T, s.d, dtype=dt, device=dev)
            self.dW1 = torch.zeros(s.d, s.E * s.f, dtype=dt, device=dev)
            self.dW2 = torch.zeros(s.E * s.f, s.d, dtype=dt, device=dev)
            self.dW3 = torch.zeros(s.d, s.E * s.f, dtype=dt, device=dev) \
                if s.act == "swiglu" else None
            self.dlogits = torch.zeros(s.T, s.E, dtype=torch.float32, device=dev)
            self.side = torch.cuda.Stream(device=dev)  # default priority
            self.ev_dyp = torch.cuda.Event()
            self.ev_dh = torch.cuda.Event()
            self.ev_wgrad = torch.cuda.Event()

    # ---------------------------------------------------------------- steps
    def _m(self, name, phase):
        if self.mark is not None:
            self.mark(name, phase)

    def _call(self, name, fn, *args, **kw):
        self._m(name, "begin")
        fn(*args, **kw)
        self._m(name, "end")

    def forward(self, x, logits, W1, W2, W3=None):
        s, t = self.s, self.topo
        c = self._call
        self.logits = logits  # the gate backward differentiates through it
        c("route_permute_topology", bsg.route_permute_topology, logits, s.k, s.renorm, self.expert_idx, self.gate,
          self.dest_row, self.counts, self.bin_offsets, self.route_ws, x, self.Tp_max,
          self.row_src, self.xp, s.f, t, bin_rows=s.bin_rows)
        if s.act == "swiglu":
            c("sdd", bsg.sdd, self.xp, W1, s.d, t, "silu_mul", self.act, b2=W3, aux_out=self.gp)
        else:
            c("sdd", bsg.sdd, self.xp, W1, s.d, t, "gelu", self.act, aux_out=self.gp)
        if self.fuse_top1:
            # Yp is kept only for the gate gradient: a forward-only layer
            # writes y alone
            c("dsd", bsg.dsd_combine_top1, self.act, t, W2, s.d, self.yp if s.backward else None,
              self.row_src, self.gate, self.y)
            return self.y
        c("dsd", bsg.dsd, self.act, t, W2, s.d, self.yp, workspace=self.dsd_ws)
        c("unpermute_combine", bsg.unpermute_combine, self.yp, self.dest_row, self.gate, s.T,
          s.k, s.d, self.y)
        return self.y

    def plane(self, blocks, i):
        """Plane i of a two-plane block array (a view)."""
        n = self.topo.nnz_max * self.block_rows
        return blocks[i * n:(i + 1) * n]

    def backward(self, dy, W1, W2, W3=None):
        s, t = self.s, self.topo
        c = self._call
        main = torch.cuda.current_stream()
        sw = s.act == "swiglu"
        dh0 = self.plane(self.dh, 0) if sw else self.dh

        def sdd_bwd():
            c("sdd_bwd", bsg.sdd, self.dyp, W2, s.d, t, "silu_mul_bwd" if sw else "gelu_bwd",
              self.dh, trans_b=True, aux_in=self.gp)

        def dsd_bwd():
            if self.fuse_top1 and not sw:  # the fused form has one block set
                c("dsd_bwd", bsg.dsd_combine_top1, self.dh, t, W1, s.d, None, self.row_src_b,
                  None, self.dx, trans_b=True)
                return
            if sw:
                c("dsd_bwd", bsg.dsd, dh0, t, W1, s.d, self.dxp, trans_b=True,
                  blocks2=self.plane(self.dh, 1), b2=W3, workspace=self.dsd_ws)
            else:
                c("dsd_bwd", bsg.dsd, self.dh, t, W1, s.d, self.dxp, trans_b=True,
                  workspace=self.dsd_ws)
            c("unpermute_combine_bwd", bsg.unpermute_combine, self.dxp, self.dest_row, None,
              s.T, s.k, s.d, self.dx)

        def dw2():
            c("dstd_dw2", bsg.dstd, self.act, t, self.dyp, s.d, self.dW2)

        def dw1():
            c("dstd_dw1", bsg.dstd, dh0, t, self.xp, s.d, self.dW1, trans_c=True)
            if sw:
                c("dstd_dw3", bsg.dstd, self.plane(self.dh, 1), t, self.xp, s.d, self.dW3,
                  trans_c=True)

        c("permute_pad_gate_bwd", bsg.permute_pad_gate_backward, dy, s.k, self.dest_row,
          self.gate, self.counts, self.bin_offsets, s.E, self.Tp_max, self.row_src_b, self.dyp,
          self.logits, s.renorm, self.expert_idx, self.yp, self.dlogits, bin_rows=s.bin_rows)
        if not self.overlap:
            sdd_bwd()
            dsd_bwd()
            dw2()
            dw1()
            return self.grads()
        self.ev_dyp.record(main)
        with torch.cuda.stream(self.side):
            self.side.wait_event(self.ev_dyp)
            dw2()
        sdd_bwd()
        self.ev_dh.record(main)
        with torch.cuda.stream(self.side):
            self.side.wait_event(self.ev_dh)
            dw1()
            self.ev_wgrad.record(self.side)
        dsd_bwd()
        main.wait_event(self.ev_wgrad)  # the step ends when both streams have
        return self.grads()

    def grads(self):
        """(dx, dW1, dW2), plus dW3 for SwiGLU experts."""
        g = (self.dx, self.dW1, self.dW2)
        return g + (self.dW3,) if self.s.act == "swiglu" else g

    def step(self, x, logits, W1, W2, W3=None, dy=None):
        """One pass of the whole hot path: forward, plus backward when set."""
        self.forward(x, logits, W1, W2, W3)
        if self.s.backward:
            self.backward(dy, W1, W2, W3)

    # ---------------------------------------------------------- helpers
    def sparse_rows(self, blocks: torch.Tensor, rows: torch.Tensor) -> torch.Tensor:
        """Gather full rows [len(rows), f] of a block-major sparse operand
        (host-side inspection helper; rows are padded-row indices)."""
        F, br = self.topo.F, self.block_rows
        b = blocks.view(-1, br, bsg.BLOCK)
        r = rows.long()
        base = (r // br) * F
        out = [b[base + j, r % br] for j in range(F)]
        return torch.cat(out, dim=1)


def from_numpy(t, dtype_str: str, device="cuda") -> torch.Tensor:
    """Upload a synth.Tensor (bf16 bit patterns or fp32 values)."""
    import numpy as np
    if dtype_str == "bf16":
        return torch.from_numpy(t.bits.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(t.values)).to(device)


def to_numpy_f64(t: torch.Tensor):
    return t.detach().float().cpu().double().numpy()
