#!/usr/bin/env python3
"""Benchmark: one step = one pass of the whole dropless-MoE hot path.

Workload (default): the MoE-Small-shaped layer, T = 32768 tokens (32 x 1024),
d = 768, E = 64 experts, f = 3072 per expert, top-1, GeLU, bf16 with fp32
accumulation, per-expert logit bias N(0, 0.5); forward + backward:
route, permute_pad, build_topology, SDD (+GeLU, keeping GeLU'), DSD, the
combine, then the dy permutation fused with the gate backward, SDD (dA *
GeLU'), DSD, the combine of dx, DSTD (dW2), DSTD (dW1).  With top-1 routing
each combine runs inside its DSD's epilogue; with k > 1 it is a launch of
its own.  ``--config mixtral_train``
runs the Mixtral-shaped SwiGLU layer (T = 8192, d = 4096, E = 8,
f = 14336, top-2) forward + backward instead.  Inputs are seeded synthetic
draws resident in HBM before the timed region.

Prints ONE JSON line.  ``value`` is the useful TFLOP/s of the step
(useful flops = 2 * T * k * d * f per product; 6 products with GeLU
experts, 9 with SwiGLU ones; padded rows are excluded).  The backward runs
the layer's schedule: the weight gradients on a second stream beside the
data-gradient chain when the products are short (MoE-Small), every call in
order on one stream otherwise; ``--overlap`` and ``--one-stream`` force
either, and ``--compare-schedules`` also times the other schedule after the
timed steps (context only).  ``roofline`` reports the step's dominant kernel
against the roof that binds it: HBM (8 TB/s) when its useful flops per
algorithmic byte fall below the ridge (2.5 PFLOP/s / 8 TB/s = 312.5), the
bf16 dense MFMA peak otherwise; its flop rate and fraction of the MFMA peak
come beside it.  The kernel's time is taken with HIP events on the stream it
runs on over the timed steps.
Which call dominates, and the per-call table ``kernels``, come from a probe
pass of three steps on one stream before the timed ones with every call
bracketed by events; the timed steps record events around the dominant call
only, since each event costs GPU time (about 4 us a call pair here).
``forward_products`` times the forward products alone (SDD + GeLU writing A
only, DSD writing Yp) with their rooflines and the ratio to a dense
hipBLASLt GEMM (torch.matmul) of the same executed shape, and the SDD with
no activation beside it (what the GeLU epilogue costs).  ``mfma_ceiling``
times the same GEMM kernel and hipBLASLt on one dense 8192^3 bf16 product
(every row in one expert): the practical MFMA ceiling beside the published
peak.
``data_movement`` times permute_pad, the backward's dy permutation with the
gate backward and unpermute_combine alone (for top-1 layers also on a top-2
routing of the same tokens), each after a 512 MiB write that flushes the
256 MB last-level cache, as GB/s of algorithmic bytes against the 8 TB/s
peak and against ``hbm_copy_ceiling``, the library's streaming copy of as
many bytes timed the same way.  ``traffic`` is HBM bytes per launch from the
committed counter summary (null once the GEMM source has changed since).
``cpu_baseline`` times the CPU oracle on a bounded sample of the same
workload on this host's cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_PEAK_BF16 = 2500.0   # TFLOP/s, dense bf16 (MI355X published figure)
MFMA_PEAK_F32 = 157.3
HBM_PEAK = 8000.0         # GB/s


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="moe_small")
    ap.add_argument("--one-stream", action="store_true",
                    help="every call in order on one stream (the layer's choice otherwise)")
    ap.add_argument("--overlap", action="store_true",
                    help="weight gradients on a second stream in the timed steps")
    ap.add_argument("--bin-rows", type=int, default=128, choices=(64, 128, 256),
                    help="pad expert bins to a multiple of this many rows (block-size study)")
    ap.add_argument("--compare-schedules", action="store_true",
                    help="after the timed steps, also time the other backward schedule")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-mfma-ceiling", action="store_true",
                    help="skip the 8192^3 dense product (context only)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle sample")
    return ap.parse_args()


def products_of(cfg, kernel):
    """GEMM products (2 * T * k * d * f useful flops each) one call performs:
    SwiGLU's forward SDD has two B operands and its input-gradient DSD two
    block sets."""
    sw = cfg.act == "swiglu"
    if kernel in ("sdd", "dsd_bwd"):
        return 2 if sw else 1
    return 1


def algorithmic_bytes(cfg, kernel, Tp, fuse_top1):
    """HBM bytes one call of a product must move at the least: each operand
    read once, each result written once (padded rows included, since they are
    stored).  Sparse planes are (Tp / 128) * F blocks of 128 x 128."""
    b = 2 if cfg.dtype == "bf16" else 4
    byp = 4 if (cfg.yp == "f32" or cfg.dtype == "f32") else 2
    sw = cfg.act == "swiglu"
    plane = Tp * cfg.f * b                                 # A, a saved factor or dH
    weight = cfg.d * cfg.E * cfg.f * b                     # W1, W2 or W3
    rows = Tp * cfg.d * b                                  # Xp or dYp
    tokens = cfg.T * cfg.d * b                             # y or dx
    if kernel == "sdd":      # rows, W1 (and W3) in; A (and the saved factors) out
        saved = (2 if sw else 1) if cfg.backward else 0
        return rows + weight * (2 if sw else 1) + plane * (1 + saved)
    if kernel == "dsd":      # A, W2 in; Yp out (and y with the top-1 combine)
        return plane + weight + Tp * cfg.d * byp + (tokens if fuse_top1 else 0)
    if kernel == "sdd_bwd":  # dYp, W2, the saved factors in; dH out
        return rows + weight + 2 * plane * (2 if sw else 1)
    if kernel == "dsd_bwd":  # dH, W1 (and W3) in; dXp out, or dx with the top-1 combine
        out = tokens if (fuse_top1 and not sw) else Tp * cfg.d * byp
        return (plane + weight) * (2 if sw else 1) + out
    if kernel.startswith("dstd"):  # blocks, dense rows in; a weight gradient out
        return plane + rows + weight
    return None


def useful_flops(cfg):
    per = 2.0 * cfg.T * cfg.k * cfg.d * cfg.f
    sw = cfg.act == "swiglu"
    products = 3 if sw else 2
    if cfg.backward:  # backward SDD, input-gradient DSD(s), one DSTD per weight
        products += 6 if sw else 4
    return per, per * products


def cpu_baseline(cfg, inp, target_s):
    """Time the oracle (as it stands) on a bounded token sample: forward
    (2 products) and the input-gradient path (2 products) per token."""
    from oracle import oracle as orc
    from block_sparse_gemm_amd import synth
    r = orc.route(inp["logits"], cfg.k, cfg.renorm, cfg.bin_rows)
    O = orc.make_layer(inp["x"].values, inp["W1"].values, inp["W2"].values, r, cfg.k, cfg.E,
                       act=cfg.act, W3=inp["W3"].values if "W3" in inp else None,
                       dy=inp["dy"].values if "dy" in inp else None, prec=cfg.dtype,
                       prec_yp=cfg.yp)
    sw = cfg.act == "swiglu"
    fwd_p, bwd_p = (3, 3) if sw else (2, 2)
    per_tok = 2.0 * cfg.k * cfg.d * cfg.f * (fwd_p + (bwd_p if cfg.backward else 0))

    def run(n):
        toks = synth.sample_tokens(cfg.T, n, seed=7)
        t0 = time.perf_counter()
        O.forward_tokens(toks)
        if cfg.backward:
            O.backward_tokens(toks)
        return len(toks), time.perf_counter() - t0

    n0, t0 = run(32)
    n = int(min(cfg.T, max(32, n0 * target_s / max(t0, 1e-3))))
    n, t = run(n)
    threads = orc.get_threads()
    # the same oracle on one core, on a sample of about a tenth of the time
    orc.set_threads(1)
    try:
        n1, t1 = run(8)
        n1, t1 = run(int(min(cfg.T, max(8, n1 * target_s / 10 / max(t1, 1e-3)))))
    finally:
        orc.set_threads(threads)
    cpu = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": per_tok * n / t / 1e12, "unit": "TFLOP/s", "cores": threads,
            "single_core_value": per_tok * n1 / t1 / 1e12,
            "single_core_sample": f"{n1} tokens, {t1:.1f} s wall on 1 thread",
            "kind": "oracle", "cpu": cpu, "affinity_cpus": len(os.sched_getaffinity(0)),
            "sample": f"{n} tokens of the {cfg.name} workload, forward"
                      + (f" + input-gradient path ({fwd_p + bwd_p} of the "
                         f"{fwd_p + bwd_p + (3 if sw else 2)} products per token; weight "
                         f"gradients not sampled)" if cfg.backward else "")
                      + f", {t:.1f} s wall on {threads} OpenMP threads"}


def traffic_for(config, kernel_name):
    """HBM bytes per launch from the committed rocprofv3 PMC summary of this
    workload, valid only while the kernel source is unchanged since the
    counters were taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{config}.json")
    if not os.path.exists(path):
        return None
    try:
        from block_sparse_gemm_amd.traffic import source_sha
        data = json.load(open(path))
        ent = data.get(kernel_name)
        if not ent or ent.get("source_sha") != source_sha():
            return None
        return ent.get("bytes_per_launch")
    except Exception:
        return None


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): the layer's "
              "multi-GPU sharding (expert parallelism over RCCL) is not built.", file=sys.stderr)
        sys.exit(2)
    import torch
    from block_sparse_gemm_amd import bsg, layer, synth

    cfg = synth.CONFIGS[args.config]
    if args.bin_rows != cfg.bin_rows:
        cfg = cfg.replace(name=f"{cfg.name}_bins{args.bin_rows}", bin_rows=args.bin_rows)
    print(f"[bench] generating inputs for {cfg.name}", file=sys.stderr, flush=True)
    inp = synth.make_inputs(cfg, 0)
    s = layer.Shape.of(cfg)
    L = layer.Layer(s)
    if args.overlap or args.one_stream:
        L.overlap = args.overlap
    two = L.overlap  # the schedule of the timed steps
    up = lambda key: layer.from_numpy(inp[key], cfg.dtype) if key in inp else None
    x, W1, W2, W3, dy = up("x"), up("W1"), up("W2"), up("W3"), up("dy")
    logits = torch.from_numpy(inp["logits"]).cuda()
    torch.cuda.synchronize()

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        L.step(x, logits, W1, W2, W3, dy)
    torch.cuda.synchronize()

    # per-call event pairs, each recorded on the stream the call runs on
    def recorder(store, only=None):
        def mark(name, phase):
            if only is None or name == only:
                ev = torch.cuda.Event(enable_timing=True)
                ev.record()
                store.append((name, phase, ev))
        return mark

    def durations(store):
        per, open_ev = {}, {}
        for name, phase, ev in store:
            if phase == "begin":
                open_ev[name] = ev
            else:
                per.setdefault(name, []).append(open_ev.pop(name).elapsed_time(ev))
        return {k: float(np.mean(v)) for k, v in per.items()}

    # probe: every call timed alone for a few steps (the per-call table, and
    # which product dominates), every call in order on one stream so that each
    # time is the call's own, not shared with a call on the other stream.
    # Events cost a few microseconds of GPU time each, so the timed steps
    # below (in the layer's schedule) record them around that product only.
    probe = []
    L.mark = recorder(probe)
    L.overlap = False
    for _ in range(3):
        L.step(x, logits, W1, W2, W3, dy)
    torch.cuda.synchronize()
    L.overlap = two
    kern = durations(probe)
    gemms = [k for k in kern if k.startswith(("sdd", "dsd", "dstd"))]
    dom = max(gemms, key=lambda k: kern[k])

    timed = []
    L.mark = recorder(timed, only=dom)
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        L.step(x, logits, W1, W2, W3, dy)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    L.mark = None
    dom_ms = durations(timed)[dom]
    step_ms = wall * 1e3 / args.steps

    # spread of the step time: a few more steps, each between two events
    NS = max(10, args.steps)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(NS + 1)]
    ev[0].record()
    for i in range(NS):
        L.step(x, logits, W1, W2, W3, dy)
        ev[i + 1].record()
    torch.cuda.synchronize()
    spread = np.percentile([ev[i].elapsed_time(ev[i + 1]) for i in range(NS)], [10, 50, 90])

    es = 2 if cfg.dtype == "bf16" else 4
    Tp = int(L.bin_offsets[-1].item())
    t = L.topo
    A_n = cfg.T * cfg.k
    ypes = 4 if (cfg.yp == "f32" or cfg.dtype == "f32") else 2

    def event_ms(fn, iters, before=None):
        """Median ms of fn over iters runs, each between two events on the
        current stream; before() runs untimed ahead of each."""
        ms = []
        for _ in range(iters):
            if before is not None:
                before()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            e1.synchronize()
            ms.append(e0.elapsed_time(e1))
        return float(np.median(ms))

    # last-level cache flush: the library's streaming copy writes (and reads)
    # 512 MiB, twice the 256 MB MALL, before each timed data-movement call
    fl_a = torch.empty(256 << 20, dtype=torch.bfloat16, device="cuda")
    fl_b = torch.empty_like(fl_a)
    flush = lambda: bsg.stream_copy(fl_a, fl_b)

    def copy_gbps(moved):
        """The library's streaming copy moving `moved` bytes (half read, half
        written), MALL flushed before each run: the HBM ceiling."""
        n = max(16, moved // 2 // 16 * 16)
        a = torch.empty(n // 2, dtype=torch.bfloat16, device="cuda")
        b = torch.empty_like(a)
        bsg.stream_copy(a, b)
        ms = event_ms(lambda: bsg.stream_copy(a, b), 10, flush)
        del a, b
        return 2 * n / (ms * 1e-3) / 1e9

    # data-movement calls alone, MALL flushed before each run
    dm = {}
    perm_bytes = cfg.T * cfg.d * es + Tp * cfg.d * es + 4 * A_n + 4 * Tp
    ceiling = copy_gbps(perm_bytes)
    big_ceiling = copy_gbps(2 << 30)
    logits_t = logits

    def entry(ms, nbytes):
        g = nbytes / (ms * 1e-3) / 1e9
        return {"ms": round(ms, 4), "bytes": int(nbytes), "gbps": round(g, 1),
                "pct_hbm_peak": round(100 * g / HBM_PEAK, 1),
                "frac_of_copy": round(g / ceiling, 3)}

    dm["permute_pad"] = entry(event_ms(lambda: bsg.permute_pad(
        x, cfg.k, L.dest_row, None, L.counts, L.bin_offsets, cfg.E, L.Tp_max, L.row_src, L.xp,
        bin_rows=cfg.bin_rows), 10, flush), perm_bytes)
    if cfg.backward:
        gb_bytes = (cfg.T * cfg.d * es + A_n * cfg.d * ypes + Tp * cfg.d * es
                    + 8 * cfg.T * cfg.E + 12 * A_n + 4 * Tp)
        dm["permute_pad_gate_bwd"] = entry(event_ms(lambda: bsg.permute_pad_gate_backward(
            dy, cfg.k, L.dest_row, L.gate, L.counts, L.bin_offsets, cfg.E, L.Tp_max,
            L.row_src_b, L.dyp, logits_t, cfg.renorm, L.expert_idx, L.yp, L.dlogits,
            bin_rows=cfg.bin_rows), 10, flush), gb_bytes)
    dm["unpermute_combine"] = entry(event_ms(lambda: bsg.unpermute_combine(
        L.yp, L.dest_row, L.gate, cfg.T, cfg.k, cfg.d, L.y), 10, flush),
        A_n * cfg.d * ypes + cfg.T * cfg.d * es + 8 * A_n)
    if cfg.k == 1:
        # the layer runs its top-1 combine inside the DSD; the standalone call
        # is also measured on a top-2 routing of the same tokens and logits
        k2 = 2
        i32 = dict(dtype=torch.int32, device="cuda")
        ei2, de2 = torch.zeros(cfg.T * k2, **i32), torch.zeros(cfg.T * k2, **i32)
        g2 = torch.zeros(cfg.T * k2, device="cuda")
        c2, b2 = torch.zeros(cfg.E, **i32), torch.zeros(cfg.E + 1, **i32)
        ws2 = torch.zeros(bsg.route_workspace_bytes(cfg.T, k2, cfg.E), dtype=torch.uint8,
                          device="cuda")
        bsg.route(logits_t, k2, False, ei2, g2, de2, c2, b2, ws2)
        Tp2 = bsg.max_padded_rows(cfg.T, k2, cfg.E)
        yp2 = torch.randn(Tp2, cfg.d, device="cuda").to(L.yp.dtype)
        dm["unpermute_combine_top2"] = entry(event_ms(lambda: bsg.unpermute_combine(
            yp2, de2, g2, cfg.T, k2, cfg.d, L.y), 10, flush),
            cfg.T * k2 * cfg.d * ypes + cfg.T * cfg.d * es + 8 * cfg.T * k2)
        del ei2, de2, g2, c2, b2, ws2, yp2
    copy_ceiling = {"kernel": "bsg_stream_copy", "same_bytes_as_permute_pad": {
        "bytes": perm_bytes, "gbps": round(ceiling, 1),
        "pct_hbm_peak": round(100 * ceiling / HBM_PEAK, 1)},
        "2GiB": {"bytes": 2 << 30, "gbps": round(big_ceiling, 1),
                 "pct_hbm_peak": round(100 * big_ceiling / HBM_PEAK, 1)},
        "flush": "512 MiB streaming copy before each timed run"}
    del fl_a, fl_b

    # forward-only products at this shape (what the layer runs without a
    # backward): SDD + GeLU writing A only, and DSD writing Yp, each against
    # its rooflines and a dense hipBLASLt GEMM (torch.matmul) of the same
    # executed shape (Tp x d x f)
    per_product = 2.0 * cfg.T * cfg.k * cfg.d * cfg.f
    peak = MFMA_PEAK_BF16 if cfg.dtype == "bf16" else MFMA_PEAK_F32
    plane = Tp * cfg.f * es
    weight = cfg.d * cfg.E * cfg.f * es
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32

    def dense_ms(M, K, N):
        a = torch.randn(M, K, device="cuda").to(dt)
        b = torch.randn(K, N, device="cuda").to(dt)
        torch.matmul(a, b)
        ms = event_ms(lambda: torch.matmul(a, b), 20)
        del a, b
        return ms

    fwd = {}
    if cfg.act == "gelu":
        W1f, W2f = W1, W2
        sdd_dense = dense_ms(Tp, cfg.d, cfg.f)
        prods = {
            "sdd_gelu": (lambda: bsg.sdd(L.xp, W1f, cfg.d, t, "gelu", L.act),
                         Tp * cfg.d * es + weight + plane, sdd_dense),
            # the same product with no activation: what the GeLU epilogue costs
            "sdd_no_activation": (lambda: bsg.sdd(L.xp, W1f, cfg.d, t, "none", L.act),
                                  Tp * cfg.d * es + weight + plane, sdd_dense),
            "dsd": (lambda: bsg.dsd(L.act, t, W2f, cfg.d, L.yp),
                    plane + weight + Tp * cfg.d * ypes, dense_ms(Tp, cfg.f, cfg.d)),
        }
        for name, (fn, nbytes, dms) in prods.items():
            fn()
            ms = event_ms(fn, 20)
            tf = per_product / (ms * 1e-3) / 1e12
            inten = per_product / nbytes
            att = min(peak, inten * HBM_PEAK / 1e3)
            fwd[name] = {"ms": round(ms, 4), "useful_tflops": round(tf, 1),
                         "frac_of_mfma_peak": round(tf / peak, 4),
                         "algorithmic_bytes": int(nbytes),
                         "intensity_flop_per_byte": round(inten, 1),
                         "attainable_tflops": round(att, 1),
                         "attainable_bound": "mfma" if att >= peak else "hbm",
                         "frac_of_attainable": round(tf / att, 4),
                         "dense_gemm_same_shape_ms": round(dms, 4),
                         "dense_ratio": round(dms / ms, 3)}

    # context: what the GEMM kernel and hipBLASLt reach on one large dense
    # bf16 product (8192 x 8192 x 8192, every row in one expert), the
    # practical MFMA ceiling on this GPU beside the published peak
    ceiling = None
    if cfg.dtype == "bf16" and not args.no_mfma_ceiling:
        n = 8192
        a = torch.randn(n, n, device="cuda").to(torch.bfloat16)
        b = torch.randn(n, n, device="cuda").to(torch.bfloat16)
        tc = bsg.Topology(n, 1, n)
        bsg.build_topology(torch.tensor([0, n], dtype=torch.int32, device="cuda"), 1, n, n, tc)
        c = torch.empty(n * n, dtype=torch.bfloat16, device="cuda")
        bsg.sdd(a, b, n, tc, "none", c)
        ms_ours = event_ms(lambda: bsg.sdd(a, b, n, tc, "none", c), 5)
        torch.matmul(a, b)
        ms_blas = event_ms(lambda: torch.matmul(a, b), 5)
        fl = 2.0 * n * n * n
        ceiling = {"shape_mnk": [n, n, n],
                   "sdd_tflops": round(fl / (ms_ours * 1e-3) / 1e12, 1),
                   "hipblaslt_tflops": round(fl / (ms_blas * 1e-3) / 1e12, 1),
                   "sdd_frac_of_mfma_peak": round(fl / (ms_ours * 1e-3) / 1e12 / MFMA_PEAK_BF16, 4)}
        del a, b, c, tc

    # context: the other backward schedule, a few steps after the timed region
    other = None
    if cfg.backward and args.compare_schedules:
        L.overlap = not two
        for _ in range(args.warmup):
            L.step(x, logits, W1, W2, W3, dy)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for _ in range(args.steps):
            L.step(x, logits, W1, W2, W3, dy)
        torch.cuda.synchronize()
        other = (time.perf_counter() - t1) * 1e3 / args.steps
        L.overlap = two

    per_product, total = useful_flops(cfg)
    tflops = total / (step_ms * 1e-3) / 1e12
    achieved = products_of(cfg, dom) * per_product / (dom_ms * 1e-3) / 1e12
    dom_bytes = algorithmic_bytes(cfg, dom, Tp, L.fuse_top1)
    intensity = products_of(cfg, dom) * per_product / dom_bytes
    attainable = min(peak, intensity * HBM_PEAK / 1e3)  # flop/B x GB/s -> TFLOP/s
    # the roof that binds this kernel: HBM when its useful flops per
    # algorithmic byte fall below the ridge (peak / 8 TB/s), else MFMA
    ridge = peak * 1e3 / HBM_PEAK
    hbm_bound = intensity < ridge
    dom_gbps = dom_bytes / (dom_ms * 1e-3) / 1e9

    kernels = {}
    for k, ms in kern.items():
        ent = {"ms": round(ms, 4)}
        if k in gemms:
            fl = products_of(cfg, k) * per_product
            ent["useful_tflops"] = round(fl / (ms * 1e-3) / 1e12, 1)
            ent["pct_bf16_peak"] = round(100 * fl / (ms * 1e-3) / 1e12 / peak, 1)
        elif k == "permute_pad_gate_bwd":  # + yp read, logits in, dlogits out
            ypes = 4 if (cfg.yp == "f32" or cfg.dtype == "f32") else 2
            b = (cfg.T * cfg.d * es + A_n * cfg.d * ypes + Tp * cfg.d * es + 8 * cfg.T * cfg.E
                 + 12 * A_n + 4 * Tp)
            ent["gbps"] = round(b / (ms * 1e-3) / 1e9, 1)
        elif k.startswith("permute_pad"):
            b = cfg.T * cfg.d * es + Tp * cfg.d * es + 4 * A_n + 4 * Tp
            ent["gbps"] = round(b / (ms * 1e-3) / 1e9, 1)
        elif k.startswith("unpermute_combine"):
            ypes = 4 if (cfg.yp == "f32" or cfg.dtype == "f32") else 2
            b = A_n * cfg.d * ypes + cfg.T * cfg.d * es + 8 * A_n
            ent["gbps"] = round(b / (ms * 1e-3) / 1e9, 1)
        elif k == "route_backward":
            ypes = 4 if (cfg.yp == "f32" or cfg.dtype == "f32") else 2
            b = cfg.T * cfg.d * es + A_n * cfg.d * ypes + 8 * cfg.T * cfg.E + 8 * A_n
            ent["gbps"] = round(b / (ms * 1e-3) / 1e9, 1)
        if "gbps" in ent:
            ent["pct_hbm_peak"] = round(100 * ent["gbps"] / HBM_PEAK, 1)
        kernels[k] = ent

    out = {
        "metric": "dMoE layer useful TFLOP/s + % of bf16 MFMA peak (1 GPU); tokens/s",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded N(0,1) logits" + (", per-expert bias" if cfg.bias_std else "")
                + (", hot/starved expert bias" if cfg.hot else "")
                + f", N(0,{cfg.x_std:g}) x, N(0,{cfg.w_std:g}) weights)",
        "config": {"workload": f"{cfg.name}: T={cfg.T}, d={cfg.d}, E={cfg.E}, f={cfg.f}, "
                               f"k={cfg.k}, {cfg.act}, "
                               f"{'forward+backward' if cfg.backward else 'forward'}, "
                               f"bins of {cfg.bin_rows} rows",
                   "padded_rows": Tp, "padding_frac": round(1 - A_n / Tp, 4)},
        "pct_of_bf16_peak": round(100 * tflops / peak, 2),
        # the same step counted with the padded rows the products execute
        "executed_tflops": round(total * Tp / A_n / (step_ms * 1e-3) / 1e12, 2),
        "tokens_per_s": round(cfg.T / (step_ms * 1e-3), 1),
        "roofline": {"kernel": dom, "bound": "hbm" if hbm_bound else "mfma",
                     "achieved": round(dom_gbps if hbm_bound else achieved, 1),
                     "peak": HBM_PEAK if hbm_bound else peak,
                     "unit": "GB/s" if hbm_bound else "TFLOP/s",
                     "frac": round(dom_gbps / HBM_PEAK if hbm_bound else achieved / peak, 4),
                     "traffic": traffic_for(cfg.name, dom), "ms": round(dom_ms, 4),
                     # the same kernel in flops, against the dense MFMA peak and
                     # against min(peak, intensity x 8 TB/s)
                     "useful_tflops": round(achieved, 1),
                     "frac_of_mfma_peak": round(achieved / peak, 4),
                     "algorithmic_bytes": dom_bytes,
                     "intensity_flop_per_byte": round(intensity, 1),
                     "ridge_flop_per_byte": round(ridge, 1),
                     "attainable_tflops": round(attainable, 1),
                     "frac_of_attainable": round(achieved / attainable, 4)},
        # every call timed alone in a probe pass before the timed steps
        "kernels": kernels,
        "forward_products": fwd or None,
        "mfma_ceiling": ceiling,
        "data_movement": dm,
        "hbm_copy_ceiling": copy_ceiling,
        "schedule": "two streams" if two else "one stream",
    }
    out["step_ms_p10_p50_p90"] = [round(float(v), 4) for v in spread]
    if other is not None:
        key = "ms_per_step_one_stream" if two else "ms_per_step_two_streams"
        out[key] = round(other, 4)
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(cfg, inp, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
