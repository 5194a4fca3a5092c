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
timed steps (context only).  ``roofline`` reports the step's dominant kernel against the bf16 dense MFMA
peak, timed with HIP events on the stream it runs on over the timed steps.
Which call dominates, and the per-call table ``kernels``, come from a probe
pass of three steps on one stream before the timed ones with every call bracketed by
events; the timed steps record events around the dominant call only, since
each event costs GPU time (about 4 us a call pair here).  The data-movement
calls' entries give HBM GB/s from their algorithmic bytes, as a share of the
8 TB/s peak and of ``hbm_copy_ceiling``, a device copy of as many bytes as
permute_pad moves, timed in the same run.  ``traffic`` is HBM bytes per
launch from the committed counter summary (null once the GEMM source has
changed since).
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
    ap.add_argument("--bin-rows", type=int, default=128, choices=(128, 256),
                    help="pad expert bins to a multiple of this many rows (block-size study)")
    ap.add_argument("--context", action="store_true",
                    help="also time dense bf16 GEMMs (torch.matmul) of the same (Tp, d, f)")
    ap.add_argument("--compare-schedules", action="store_true",
                    help="after the timed steps, also time the other backward schedule")
    ap.add_argument("--no-cpu-baseline", action="store_true")
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
    plane = (Tp // 128) * (cfg.f // 128) * 128 * 128 * b  # A, a saved factor or dH
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
    from block_sparse_gemm_amd import layer, synth

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

    # context: a device-to-device copy (torch copy_) moving as many bytes as
    # permute_pad reads and writes, through four rotating buffer pairs so the
    # 256 MB MALL cannot serve repeats: the practical HBM ceiling that the
    # data-movement calls are compared with
    es = 2 if cfg.dtype == "bf16" else 4
    Tp = int(L.bin_offsets[-1].item())
    half = (cfg.T + Tp) * cfg.d * es // 2
    pairs = [(torch.empty(half // 2, dtype=torch.bfloat16, device="cuda"),
              torch.empty(half // 2, dtype=torch.bfloat16, device="cuda")) for _ in range(4)]
    for i in range(4):
        pairs[i][1].copy_(pairs[i][0])
    ce0, ce1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ce0.record()
    for i in range(20):
        pairs[i % 4][1].copy_(pairs[i % 4][0])
    ce1.record()
    torch.cuda.synchronize()
    copy_gbps = 2 * (half // 2) * 2 / (ce0.elapsed_time(ce1) / 20 * 1e-3) / 1e9
    del pairs

    # context: dense bf16 GEMMs with the products' executed shapes (M = Tp)
    dense = None
    if args.context:
        Tp0 = int(L.bin_offsets[-1].item())
        dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
        a1 = torch.randn(Tp0, cfg.d, device="cuda").to(dt)
        b1 = torch.randn(cfg.d, cfg.f, device="cuda").to(dt)
        a2 = torch.randn(Tp0, cfg.f, device="cuda").to(dt)
        b2 = torch.randn(cfg.f, cfg.d, device="cuda").to(dt)

        def time_mm(a, b):
            for _ in range(3):
                torch.matmul(a, b)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(20):
                torch.matmul(a, b)
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / 20

        dense = {"sdd_shape_ms": round(time_mm(a1, b1), 4),
                 "dsd_shape_ms": round(time_mm(a2, b2), 4)}
        del a1, b1, a2, b2

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
    peak = MFMA_PEAK_BF16 if cfg.dtype == "bf16" else MFMA_PEAK_F32
    dom_bytes = algorithmic_bytes(cfg, dom, int(L.bin_offsets[-1].item()), L.fuse_top1)
    intensity = products_of(cfg, dom) * per_product / dom_bytes
    attainable = min(peak, intensity * HBM_PEAK / 1e3)  # flop/B x GB/s -> TFLOP/s

    kernels = {}
    A_n = cfg.T * cfg.k
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
            ent["frac_of_copy"] = round(ent["gbps"] / copy_gbps, 3)
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
        "roofline": {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 1),
                     "peak": peak, "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": traffic_for(cfg.name, dom), "ms": round(dom_ms, 4),
                     # the same product against min(peak, intensity x 8 TB/s):
                     # useful flops per algorithmic HBM byte decide whether
                     # matrix cores or HBM bound it at this shape
                     "algorithmic_bytes": dom_bytes,
                     "intensity_flop_per_byte": round(intensity, 1),
                     "attainable": round(attainable, 1),
                     "attainable_bound": "mfma" if attainable >= peak else "hbm",
                     "frac_of_attainable": round(achieved / attainable, 4)},
        # every call timed alone in a probe pass before the timed steps
        "kernels": kernels,
        "hbm_copy_ceiling": {"bytes": 2 * (half // 2) * 2, "gbps": round(copy_gbps, 1),
                             "pct_hbm_peak": round(100 * copy_gbps / HBM_PEAK, 1)},
        "schedule": "two streams" if two else "one stream",
    }
    out["step_ms_p10_p50_p90"] = [round(float(v), 4) for v in spread]
    if other is not None:
        key = "ms_per_step_one_stream" if two else "ms_per_step_two_streams"
        out[key] = round(other, 4)
    if dense is not None:
        # the block-sparse product's time against a dense GEMM of its executed
        # shape (Tp x d x f): the block-sparse kernel runs at ratio x the
        # dense GEMM's throughput on the same work
        fl_exec = 2.0 * Tp * cfg.d * cfg.f
        dense["sdd_ratio"] = round(dense["sdd_shape_ms"] * products_of(cfg, "sdd")
                                   / kern["sdd"], 3)
        dense["dsd_ratio"] = round(dense["dsd_shape_ms"] / kern["dsd"], 3)
        dense["dense_tflops"] = round(fl_exec / (dense["sdd_shape_ms"] * 1e-3) / 1e12, 1)
        out["context_dense_gemm"] = dense
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(cfg, inp, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
