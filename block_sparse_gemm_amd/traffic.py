"""HBM traffic per kernel launch from rocprofv3 counters, and the Markdown
summaries of rocprofv3 output kept under profiles/.

Modes:

``python3 -m block_sparse_gemm_amd.traffic run [--config moe_small] [--steps 2]``
    The workload for a counter pass: a plain copy of a known size (the
    calibration), then ``--steps`` steps of the layer.  Run it under
    ``rocprofv3 --pmc FETCH_SIZE`` and, separately, ``--pmc WRITE_SIZE``.

``python3 -m block_sparse_gemm_amd.traffic counters --csv A.csv B.csv ... --md OUT.md``
    Per call of the layer, the mean per dispatch of every counter in the given
    ``*_counter_collection.csv`` files, and the busy fractions derived from
    them on MI355X (8 XCDs, 256 CUs, 1024 SIMDs): MFMA busy, TA busy, TD busy,
    TD stalled on the L2, LDS bank-conflict share, L2 hit rate.

``python3 -m block_sparse_gemm_amd.traffic summarize --fetch F.csv --write W.csv``
    Reads the two ``*_counter_collection.csv`` files, scales each kernel's
    mean counter value per dispatch by what the copy kernel reads for its
    known byte count, and writes ``profiles/traffic_<config>.json`` (bytes
    per launch, keyed by the layer's call names, stamped with the hash of the
    GEMM source so stale figures are ignored) and a Markdown table.

``python3 -m block_sparse_gemm_amd.traffic stats --csv run_kernel_stats.csv --md OUT.md``
    The per-kernel table of a ``rocprofv3 --kernel-trace --stats`` run
    (calls, mean / min / max duration, share of the traced time), with each
    GEMM instantiation named by its product, epilogue and operand layout.
"""
from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import json
import os
import re
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
# every source the GEMM kernels are compiled from, and the launch parameters
# (tile grouping) set in the C ABI
GEMM_SRCS = [os.path.join(ROOT, "block_sparse_gemm_amd", "csrc", n)
             for n in ("gemm.hpp", "gemm.hip", "gemm_br128.hip", "gemm_br64.hip", "common.hpp",
                       "kernels.hpp", "api.cpp")]
COPY_BYTES = 1 << 29           # 512 MiB read and 512 MiB written by the calibration copy
COPY_NAMES = ("copyBuffer", "MulFunctor")   # the memcpy blit kernel, else x * 1


def source_sha() -> str:
    h = hashlib.sha256()
    for path in GEMM_SRCS:
        h.update(open(path, "rb").read())
    return h.hexdigest()[:16]


def traffic_path(config: str) -> str:
    return os.path.join(ROOT, "profiles", f"traffic_{config}.json")


def call_name(kernel: str):
    """Map a kernel symbol to the layer's call name (None if not a layer kernel).

    Template arguments: dtype, mode (0 SDD, 1 dual-B SDD, 2 DSD, 3 DSTD, 4
    two-set DSD), B K-contiguous, epilogue (3 and 4: the backward ones), out
    dtype, swap (false: transposed DSTD output), block rows.  dW1 and dW3 run
    the same instantiation and share its figure."""
    m = re.search(r"dsd_reduce_kernel<(\d+), (\w+), (\d+), (\d+)>", kernel)
    if m:  # the second launch of a split DSD, named by the product it completes
        mode, b_kc = m.group(1), m.group(2)
        return "dsd_bwd" if mode == "4" or b_kc == "true" else "dsd"
    m = re.search(r"gemm_kernel<(\d+), (\d+), (\w+), (\d+), (\d+), (\w+)(?:, (\d+))?>", kernel)
    if m:
        _, mode, b_kc, epi, _, swap, _ = m.groups()
        if mode in ("0", "1"):
            return "sdd_bwd" if epi in ("3", "4") else "sdd"
        if mode == "2":
            return "dsd_bwd" if b_kc == "true" else "dsd"
        if mode == "4":
            return "dsd_bwd"
        if mode == "3":
            return "dstd_dw2" if swap == "true" else "dstd_dw1"
    if "permute_gate_backward" in kernel:
        return "permute_pad_gate_bwd"
    for k in ("route_backward", "route_topk", "route_scan", "route_place", "permute_pad",
              "build_topology", "combine"):
        if k in kernel:
            return k
    return None


def run(args):
    import torch
    from block_sparse_gemm_amd import layer, synth

    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    print("[traffic] calibration copy", flush=True)
    dst.copy_(src)
    torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    del src, dst

    cfg = synth.CONFIGS[args.config]
    inp = synth.make_inputs(cfg, 0)
    s = layer.Shape.of(cfg)
    L = layer.Layer(s)
    up = lambda key: layer.from_numpy(inp[key], cfg.dtype) if key in inp else None
    x, W1, W2, W3, dy = up("x"), up("W1"), up("W2"), up("W3"), up("dy")
    logits = torch.from_numpy(inp["logits"]).cuda()
    torch.cuda.synchronize()
    for i in range(args.steps):
        L.step(x, logits, W1, W2, W3, dy)
        torch.cuda.synchronize()
        print(f"[traffic] step {i} done", flush=True)


def per_dispatch(path):
    """{kernel name: [value per dispatch, ...]} in KiB, summed over counter instances."""
    acc = collections.defaultdict(float)
    names = {}
    for r in csv.DictReader(open(path)):
        key = r["Dispatch_Id"]
        acc[key] += float(r["Counter_Value"])
        names[key] = r["Kernel_Name"]
    out = collections.defaultdict(list)
    for key, v in acc.items():
        out[names[key]].append(v)
    return out


def summarize(args):
    fetch, write = per_dispatch(args.fetch), per_dispatch(args.write)

    def copy_factor(table, label):
        for pat in COPY_NAMES:
            cands = [v for k, vs in table.items() if pat in k for v in vs]
            if cands and max(cands) > 0:
                big = max(cands)
                return COPY_BYTES / (big * 1024.0), big
        raise SystemExit(f"no calibration copy found in the {label} counters")

    f_fac, f_raw = copy_factor(fetch, "FETCH_SIZE")
    w_fac, w_raw = copy_factor(write, "WRITE_SIZE")
    sha = source_sha()
    result = {"_calibration": {"copy_bytes": COPY_BYTES, "fetch_kib": f_raw, "write_kib": w_raw,
                               "fetch_factor": f_fac, "write_factor": w_fac,
                               "workload": args.config}}
    rows = []
    for kern in sorted(set(fetch) | set(write)):
        name = call_name(kern)
        if name is None:
            continue
        fk = sum(fetch.get(kern, [0])) / max(1, len(fetch.get(kern, [])))
        wk = sum(write.get(kern, [0])) / max(1, len(write.get(kern, [])))
        fb, wb = fk * 1024 * f_fac, wk * 1024 * w_fac
        ent = {"fetch_bytes": round(fb), "write_bytes": round(wb), "bytes_per_launch": round(fb + wb),
               "kernel": kern[:120]}
        if kern.find("gemm_kernel") >= 0 or kern.find("dsd_reduce_kernel") >= 0:
            ent["source_sha"] = sha
        if name in result:  # a call of two launches (a split DSD): per call, both
            prev = result[name]
            ent = dict(prev, fetch_bytes=prev["fetch_bytes"] + ent["fetch_bytes"],
                       write_bytes=prev["write_bytes"] + ent["write_bytes"],
                       bytes_per_launch=prev["bytes_per_launch"] + ent["bytes_per_launch"],
                       kernel=prev["kernel"] + " + " + ent["kernel"][:60])
        result[name] = ent
        if name == "dstd_dw1":
            result["dstd_dw3"] = ent
        rows.append((name, fb / 1e6, wb / 1e6, kern[:80]))
    out = args.out or traffic_path(args.config)
    md = args.md or os.path.join(ROOT, "profiles", f"{args.config}_traffic.md")
    os.makedirs(os.path.dirname(out), exist_ok=True)
    json.dump(result, open(out, "w"), indent=1)
    lines = [f"# HBM traffic per launch: {args.config} layer step", "",
             "Counters FETCH_SIZE and WRITE_SIZE (KiB per dispatch, summed over L2 channels), each scaled",
             f"by the reading of a plain {COPY_BYTES >> 20} MiB copy: fetch factor {f_fac:.4f}, write factor "
             f"{w_fac:.4f}.", "", "Commands:", "", "```"] + args.cmd + ["```", "",
             "| call | fetch MB | write MB | kernel |", "|---|---|---|---|"]
    for name, fm, wm, k in rows:
        lines.append(f"| {name} | {fm:.1f} | {wm:.1f} | `{k}` |")
    open(md, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


XCDS, CUS, SIMDS = 8, 256, 1024   # MI355X


def counters(args):
    table = collections.defaultdict(lambda: collections.defaultdict(list))
    for path in args.csv:
        per = collections.defaultdict(lambda: collections.defaultdict(float))
        names = {}
        for r in csv.DictReader(open(path)):
            per[r["Dispatch_Id"]][r["Counter_Name"]] += float(r["Counter_Value"])
            names[r["Dispatch_Id"]] = r["Kernel_Name"]
        for disp, cs in per.items():
            name = call_name(names[disp])
            if name is None:
                continue
            cyc = cs.get("GRBM_GUI_ACTIVE", 0.0) / XCDS
            for c, v in cs.items():
                table[name][c].append(v)
            if cyc <= 0:
                continue
            derived = {
                "MFMA busy": ("SQ_VALU_MFMA_BUSY_CYCLES", SIMDS),
                "TA busy": ("TA_BUSY_avr", 1),
                "TD busy": ("TD_TD_BUSY", CUS),
                "TD stalled on L2": ("TD_TC_STALL", CUS),
                "TA stalled on L2": ("TA_ADDR_STALLED_BY_TC_CYCLES", CUS),
            }
            for label, (c, n) in derived.items():
                if c in cs:
                    table[name]["% " + label].append(100.0 * cs[c] / (n * cyc))
            if cs.get("SQ_LDS_IDX_ACTIVE"):
                table[name]["% LDS bank conflict"].append(
                    100.0 * cs.get("SQ_LDS_BANK_CONFLICT", 0.0) / cs["SQ_LDS_IDX_ACTIVE"])
            hit, miss = cs.get("TCC_HIT_sum"), cs.get("TCC_MISS_sum")
            if hit is not None and miss is not None and hit + miss > 0:
                table[name]["% L2 hit"].append(100.0 * hit / (hit + miss))
    cols = sorted({c for cs in table.values() for c in cs if c.startswith("% ")})
    order = ["sdd", "dsd", "sdd_bwd", "dsd_bwd", "dstd_dw2", "dstd_dw1", "permute_pad",
             "permute_pad_gate_bwd", "combine"]
    calls = [c for c in order if c in table] + sorted(c for c in table if c not in order)
    lines = [f"# Counters per call: {args.config} layer step", "",
             "Busy fractions of the kernel's active cycles (GRBM_GUI_ACTIVE per XCD), normalised by",
             f"the unit count on MI355X ({SIMDS} SIMDs for MFMA, {CUS} CUs for TD, TA_BUSY_avr already",
             "averaged); LDS bank conflict = SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE; L2 hit =",
             "TCC_HIT_sum / (TCC_HIT_sum + TCC_MISS_sum).  Means over the profiled dispatches.", "",
             "Commands:", "", "```"] + args.cmd + ["```", "",
             "| call | " + " | ".join(c[2:] + " %" for c in cols) + " |",
             "|---|" + "---|" * len(cols)]
    for name in calls:
        vals = [table[name].get(c) for c in cols]
        lines.append(f"| {name} | " + " | ".join(
            "—" if not v else f"{sum(v) / len(v):.1f}" for v in vals) + " |")
    open(args.md, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


_MODES = {"0": "sdd", "1": "sdd_dual", "2": "dsd", "3": "dstd", "4": "dsd_two_sets"}
_EPIS = {"0": "", "1": "+gelu", "2": "+silu_mul", "3": "+gelu_bwd", "4": "+silu_mul_bwd",
         "5": "+gelu (saves gelu')", "6": "+silu_mul (saves silu, u*silu')", "7": "+top-1 combine"}


def kernel_label(name: str) -> str:
    """A readable name for a kernel of the stats table: GEMM instantiations
    by product, epilogue, B operand layout and output type."""
    m = re.match(r"void bsg::gemm_kernel<(\d+), (\d+), (\w+), (\d+), (\d+), (\w+)(?:, (\d+))?>",
                 name)
    if m:
        _, mode, bk, epi, out, swap, br = m.groups()
        return (f"gemm {_MODES.get(mode, mode)}{_EPIS.get(epi, '+' + epi)} "
                f"(B {'K' if bk == 'true' else 'MN'}-contig, out {'bf16' if out == '1' else 'f32'}"
                f"{'' if swap == 'true' else ', transposed'}"
                f"{', blocks of ' + br + ' rows' if br and br != '128' else ''})")
    m = re.match(r"void bsg::dsd_reduce_kernel<(\d+), (\w+), (\d+), (\d+)>", name)
    if m:
        mode, bk, out, br = m.groups()
        return (f"split-DSD sum of shares ({_MODES.get(mode, mode)}, B "
                f"{'K' if bk == 'true' else 'MN'}-contig, out {'bf16' if out == '1' else 'f32'}"
                f"{', blocks of ' + br + ' rows' if br != '128' else ''})")
    return re.sub(r"\(.*", "", name).replace("void ", "")[:70]


def stats(args):
    rows = list(csv.DictReader(open(args.csv)))
    lines = [f"# {args.title}", "", "Command (run from the repository root on one MI355X):", "",
             "```"] + args.cmd + ["```", "",
             "| kernel | calls | avg us | min us | max us | share |", "|---|---|---|---|---|---|"]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        lines.append(f"| {kernel_label(r['Name'])} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} "
                     f"| {float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} "
                     f"| {float(r['Percentage']):.1f}% |")
    open(args.md, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="mode", required=True)
    r = sub.add_parser("run")
    r.add_argument("--config", default="moe_small")
    r.add_argument("--steps", type=int, default=2)
    s = sub.add_parser("summarize")
    s.add_argument("--fetch", required=True)
    s.add_argument("--write", required=True)
    s.add_argument("--config", default="moe_small")
    s.add_argument("--out", default=None, help="default profiles/traffic_<config>.json")
    s.add_argument("--md", default=None, help="default profiles/<config>_traffic.md")
    s.add_argument("--cmd", nargs="*", default=[])
    c = sub.add_parser("counters")
    c.add_argument("--csv", nargs="+", required=True)
    c.add_argument("--config", default="moe_small")
    c.add_argument("--md", required=True)
    c.add_argument("--cmd", nargs="*", default=[])
    k = sub.add_parser("stats")
    k.add_argument("--csv", required=True, help="rocprofv3 run_kernel_stats.csv")
    k.add_argument("--md", required=True)
    k.add_argument("--title", required=True)
    k.add_argument("--cmd", nargs="*", default=[])
    a = ap.parse_args()
    sys.path.insert(0, ROOT)
    {"run": run, "summarize": summarize, "counters": counters, "stats": stats}[a.mode](a)


if __name__ == "__main__":
    main()
