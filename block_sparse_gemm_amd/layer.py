"""The dropless-MoE expert layer as a chain of the library's calls.

Forward (George Lin's Blog, MegaBlocks/FlexMoE post, sections 1.2-1.4):
    route -> permute_pad -> build_topology -> sdd (+ activation) -> dsd
    -> unpermute_combine
Backward (plain calculus on the same products, weight gradients through the
transpose index as section 1.3 describes):
    permute_pad(dy, scale = gate) -> sdd(dYp, W2^T, GeLU') -> dsd(dH, W1^T)
    -> unpermute_combine(gate = 1) ; dstd(A, dYp) = dW2 ; dstd(dH, Xp)^T = dW1 ;
    route_backward(dy, Yp) = dlogits (the gate's gradient, selection fixed)
The two weight gradients run on a second stream, each as soon as its inputs
exist (dW2 beside the GeLU' product, dW1 beside the input-gradient product),
so the tail of one product's grid and the other's fill the GPU together.

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
        # weight gradients on the second stream (False: everything in order
        # on the caller's stream, e.g. to time each call alone)
        self.overlap = True
        dev = torch.device(device)
        i32 = dict(dtype=torch.int32, device=dev)
        A = s.T * s.k
        self.Tp_max = bsg.max_padded_rows(s.T, s.k, s.E)
        self.topo = bsg.Topology(self.Tp_max, s.E, s.f, device=dev)
        nnz_max = self.topo.nnz_max
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
        self.act = torch.zeros(nnz_max * bsg.BLOCK, bsg.BLOCK, dtype=dt, device=dev)
        # what the backward keeps of the forward: GeLU'(h), block-major like A
        self.gp = torch.zeros_like(self.act) if s.backward else None
        self.yp = torch.zeros(self.Tp_max, s.d, dtype=ydt, device=dev)
        self.y = torch.zeros(s.T, s.d, dtype=dt, device=dev)
        if s.backward:
            if s.act != "gelu":
                raise NotImplementedError("backward is implemented for GeLU experts")
            self.dyp = torch.zeros(self.Tp_max, s.d, dtype=dt, device=dev)
            self.row_src_b = torch.zeros(self.Tp_max, **i32)
            self.dh = torch.zeros_like(self.act)
            self.dxp = torch.zeros(self.Tp_max, s.d, dtype=ydt, device=dev)
            self.dx = torch.zeros(s.T, s.d, dtype=dt, device=dev)
            self.dW1 = torch.zeros(s.d, s.E * s.f, dtype=dt, device=dev)
            self.dW2 = torch.zeros(s.E * s.f, s.d, dtype=dt, device=dev)
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
        c("route", bsg.route, logits, s.k, s.renorm, self.expert_idx, self.gate, self.dest_row,
          self.counts, self.bin_offsets, self.route_ws)
        c("permute_pad", bsg.permute_pad, x, s.k, self.dest_row, None, self.counts,
          self.bin_offsets, s.E, self.Tp_max, self.row_src, self.xp)
        c("build_topology", bsg.build_topology, self.bin_offsets, s.E, s.f, self.Tp_max, t)
        if s.act == "swiglu":
            c("sdd", bsg.sdd, self.xp, W1, s.d, t, "silu_mul", self.act, b2=W3)
        else:
            c("sdd", bsg.sdd, self.xp, W1, s.d, t, "gelu", self.act, aux_out=self.gp)
        c("dsd", bsg.dsd, self.act, t, W2, s.d, self.yp)
        c("unpermute_combine", bsg.unpermute_combine, self.yp, self.dest_row, self.gate, s.T,
          s.k, s.d, self.y)
        return self.y

    def backward(self, dy, W1, W2):
        s, t = self.s, self.topo
        c = self._call
        main = torch.cuda.current_stream()
        c("permute_pad_bwd", bsg.permute_pad, dy, s.k, self.dest_row, self.gate, self.counts,
          self.bin_offsets, s.E, self.Tp_max, self.row_src_b, self.dyp)
        if not self.overlap:
            c("route_backward", bsg.route_backward, self.logits, s.k, s.renorm, self.expert_idx,
              self.dest_row, dy, self.yp, self.dlogits)
            c("sdd_bwd", bsg.sdd, self.dyp, W2, s.d, t, "gelu_bwd", self.dh, trans_b=True,
              aux_in=self.gp)
            c("dsd_bwd", bsg.dsd, self.dh, t, W1, s.d, self.dxp, trans_b=True)
            c("unpermute_combine_bwd", bsg.unpermute_combine, self.dxp, self.dest_row, None,
              s.T, s.k, s.d, self.dx)
            c("dstd_dw2", bsg.dstd, self.act, t, self.dyp, s.d, self.dW2)
            c("dstd_dw1", bsg.dstd, self.dh, t, self.xp, s.d, self.dW1, trans_c=True)
            return self.dx, self.dW1, self.dW2
        self.ev_dyp.record(main)
        with torch.cuda.stream(self.side):
            self.side.wait_event(self.ev_dyp)
            c("route_backward", bsg.route_backward, self.logits, s.k, s.renorm, self.expert_idx,
              self.dest_row, dy, self.yp, self.dlogits)
            c("dstd_dw2", bsg.dstd, self.act, t, self.dyp, s.d, self.dW2)
        c("sdd_bwd", bsg.sdd, self.dyp, W2, s.d, t, "gelu_bwd", self.dh, trans_b=True,
          aux_in=self.gp)
        self.ev_dh.record(main)
        with torch.cuda.stream(self.side):
            self.side.wait_event(self.ev_dh)
            c("dstd_dw1", bsg.dstd, self.dh, t, self.xp, s.d, self.dW1, trans_c=True)
            self.ev_wgrad.record(self.side)
        c("dsd_bwd", bsg.dsd, self.dh, t, W1, s.d, self.dxp, trans_b=True)
        c("unpermute_combine_bwd", bsg.unpermute_combine, self.dxp, self.dest_row, None, s.T,
          s.k, s.d, self.dx)
        main.wait_event(self.ev_wgrad)  # the step ends when both streams have
        return self.dx, self.dW1, self.dW2

    def step(self, x, logits, W1, W2, W3=None, dy=None):
        """One pass of the whole hot path: forward, plus backward when set."""
        self.forward(x, logits, W1, W2, W3)
        if self.s.backward:
            self.backward(dy, W1, W2)

    # ---------------------------------------------------------- helpers
    def sparse_rows(self, blocks: torch.Tensor, rows: torch.Tensor) -> torch.Tensor:
        """Gather full rows [len(rows), f] of a block-major sparse operand
        (host-side inspection helper; rows are padded-row indices)."""
        F = self.topo.F
        b = blocks.view(-1, bsg.BLOCK, bsg.BLOCK)
        r = rows.long()
        base = (r // bsg.BLOCK) * F
        out = [b[base + j, r % bsg.BLOCK] for j in range(F)]
        return torch.cat(out, dim=1)


def from_numpy(t, dtype_str: str, device="cuda") -> torch.Tensor:
    """Upload a synth.Tensor (bf16 bit patterns or fp32 values)."""
    import numpy as np
    if dtype_str == "bf16":
        return torch.from_numpy(t.bits.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(t.values)).to(device)


def to_numpy_f64(t: torch.Tensor):
    return t.detach().float().cpu().double().numpy()
