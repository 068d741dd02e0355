"""Profiling helpers for rocprofv3 runs of the MoE layer.

    # the workload to profile (run it under rocprofv3):
    python -m mixture_experts_layer_deepseekmoe_amd.profiling run --workload bf16_d7168 --steps 3
    # measured ceilings (MFMA with random / zero operands, HBM stream) -> profiles/measured_peaks.json:
    python -m mixture_experts_layer_deepseekmoe_amd.profiling peaks
    # the vendor library (hipBLASLt through torch) on GEMMs of the same sizes -> profiles/library_reference.json:
    python -m mixture_experts_layer_deepseekmoe_amd.profiling library --workload bf16_d7168
    # turn rocprofv3's CSV output into the summaries kept under profiles/:
    python -m mixture_experts_layer_deepseekmoe_amd.profiling summarize --trace DIR --pmc DIR [DIR...] \
        --workload bf16_d7168 --out profiles

``run`` first launches one plain streaming kernel of known size (an fp64
elementwise multiply of a 1 GiB tensor into another: 1 GiB read, 1 GiB
written; nothing else in the run is fp64), which calibrates the HBM byte
counters (FETCH_SIZE / WRITE_SIZE), then a few layer forwards.  ``summarize`` averages every counter per kernel
and per dispatch, scales FETCH_SIZE / WRITE_SIZE by the calibration, and
writes a markdown summary plus profiles/traffic_counters.json.
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys
from collections import defaultdict

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CALIB_BYTES = 1 << 30


def _run(args):
    sys.path.insert(0, ROOT)
    import torch

    import mixture_experts_layer_deepseekmoe_amd as moe
    from moe_workloads import get_config, make_inputs

    torch.cuda.set_device(0)
    src = torch.ones(CALIB_BYTES // 8, dtype=torch.float64, device="cuda")
    dst = torch.empty_like(src)
    torch.mul(src, 2.0, out=dst)
    torch.cuda.synchronize()
    del src, dst

    cfg = get_config(args.workload)
    inp = make_inputs(cfg, 0, weights_device="cuda")
    shape = moe.LayerShape.from_config(cfg)
    u, cen, bias = (t.cuda().contiguous() for t in (inp.u, inp.centroids, inp.bias))
    w = moe.prepare_weights(cfg, inp, train=args.train)
    ws = moe.alloc_workspace(shape)
    routing = moe.alloc_routing(shape)
    y = torch.empty((cfg.T, cfg.d), dtype=torch.float32 if cfg.out_dtype == "f32" else torch.bfloat16, device="cuda")
    if args.train:
        tws = moe.alloc_train_workspace(shape)
        g = torch.Generator(device="cuda")
        g.manual_seed(7)
        dy = torch.randn((cfg.T, cfg.d), generator=g, device="cuda", dtype=torch.float32)
        grads = moe.alloc_weight_grads(shape)
    for i in range(args.steps):
        if args.train:
            moe.moe_forward_train(shape, u, cen, bias, w, tws, y=y)
            moe.moe_backward(shape, u, cen, w, dy, tws, grads=grads)
        else:
            moe.moe_forward(shape, u, cen, bias, w, y=y, routing=routing, workspace=ws)
            moe.moe_update_bias(bias, routing["expert_counts"], cfg.T * cfg.top_k)
        torch.cuda.synchronize()
        print(f"[profile] step {i} done", flush=True)


def _short(name: str) -> str:
    for key in ("dgrad_down_kernel", "dgrad_gateup_kernel", "wgrad_down_kernel", "wgrad_gateup_kernel",
                "wgrad8_down_kernel", "wgrad8_gateup_kernel", "colquant_kernel", "swiglu_bwd_kernel",
                "bwd_prep_kernel", "bwd_dz_kernel", "bwd_du_kernel", "bwd_de_kernel",
                "gateup_kernel", "down_kernel", "route_part_kernel", "route_finish_kernel", "route_scores_kernel",
                "route_topk_kernel", "route_kernel", "combine_kernel", "hist_kernel", "scan_kernel",
                "permute_kernel", "quant_act_kernel", "quant_weight_kernel", "bias_update_kernel"):
        if key in name:
            fmt = ""
            if "ILi1E" in name:
                fmt = "<bf16>"
            elif "ILi2E" in name:
                fmt = "<e4m3>"
            elif "ILi0E" in name:
                fmt = "<f32>"
            return key + fmt
    if name.startswith("void at::native::"):
        return "torch:" + name[len("void at::native::"):].split("<")[0].split("(")[0]
    return name[:60]


CALIB = "calibration_stream(1GiB read + 1GiB write)"


def _is_calibration(row) -> bool:
    # the fp64 multiply of the 1 GiB calibration tensor
    return "MulFunctor<double>" in row["Kernel_Name"]


# rocprofv3 --kernel-include-regex for counter runs: the layer's kernels and
# the calibration stream (keeps the input generators' kernels out of the CSV)
KERNEL_REGEX = ("gateup_kernel|down_kernel|route_kernel|route_part_kernel|route_finish_kernel|combine_kernel|"
                "hist_kernel|scan_kernel|permute_kernel|quant_act_kernel|bias_update_kernel|bwd_prep_kernel|"
                "bwd_dz_kernel|bwd_du_kernel|bwd_de_kernel|colquant_kernel|swiglu_bwd_kernel|MulFunctor<double>")


def _csvs(d, pattern):
    return sorted(glob.glob(os.path.join(d, "**", pattern), recursive=True))


def kernel_stats(trace_dir):
    rows = []
    for f in _csvs(trace_dir, "*kernel_stats.csv"):
        rows += list(csv.DictReader(open(f)))
    return rows


def counters(pmc_dirs):
    """{kernel: {counter: mean value per dispatch}}"""
    acc = defaultdict(lambda: defaultdict(list))
    for d in pmc_dirs:
        for f in _csvs(d, "*counter_collection.csv"):
            per = defaultdict(float)
            for r in csv.DictReader(open(f)):
                name = CALIB if _is_calibration(r) else _short(r["Kernel_Name"])
                key = (r["Dispatch_Id"], name, r["Counter_Name"])
                per[key] += float(r["Counter_Value"])
            for (disp, k, c), v in per.items():
                acc[k][c].append(v)
    return {k: {c: sum(v) / len(v) for c, v in cs.items()} for k, cs in acc.items()}


def source_hash(train: bool = False):
    """Hash of the grouped-GEMM sources (with ``train``, the backward's too),
    stamped on stored counter readings."""
    csrc = os.path.join(ROOT, "mixture_experts_layer_deepseekmoe_amd", "csrc")
    h = hashlib.sha256()
    files = ["gemm_core.hpp", "ggemm.hip", "tile_map.hpp", "moe_common.hpp", "kernels.hpp"]
    for f in files + (["bwd.hip"] if train else []):
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def _summarize(args):
    os.makedirs(args.out, exist_ok=True)
    lines = [f"# rocprofv3 summary: {args.workload}", ""]
    if args.command:
        lines += ["Commands:", ""] + [f"    {c}" for c in args.command] + [""]
    ks = kernel_stats(args.trace) if args.trace else []
    if ks:
        lines += ["## Kernel trace (--kernel-trace --stats)", "",
                  "| kernel | calls | total ms | avg us | min us | max us | % |", "|---|---|---|---|---|---|---|"]
        for r in ks:
            name = _short(r.get("Name", r.get("KernelName", "")))
            calls = int(r.get("Calls", 0))
            tot = float(r.get("TotalDurationNs", 0)) / 1e6
            avg = float(r.get("AverageNs", 0)) / 1e3
            mn = float(r.get("MinNs", 0)) / 1e3
            mx = float(r.get("MaxNs", 0)) / 1e3
            pct = float(r.get("Percentage", 0))
            lines.append(f"| {name} | {calls} | {tot:.3f} | {avg:.1f} | {mn:.1f} | {mx:.1f} | {pct:.2f} |")
        lines.append("")
    traffic = None
    if args.pmc:
        cs = counters(args.pmc)
        cal = cs.get(CALIB, {})
        fetch_f = CALIB_BYTES / (cal["FETCH_SIZE"] * 1024) if cal.get("FETCH_SIZE") else None
        write_f = CALIB_BYTES / (cal["WRITE_SIZE"] * 1024) if cal.get("WRITE_SIZE") else None
        lines += ["## Counters (mean per dispatch)", "",
                  f"Calibration: a streaming kernel that reads and writes {CALIB_BYTES} bytes each reads "
                  f"FETCH_SIZE = {cal.get('FETCH_SIZE', float('nan')):.0f} KiB and WRITE_SIZE = "
                  f"{cal.get('WRITE_SIZE', float('nan')):.0f} KiB; scale factors fetch {fetch_f}, write {write_f}.", ""]
        names = sorted({c for v in cs.values() for c in v})
        lines += ["| kernel | " + " | ".join(names) + " |", "|---" * (len(names) + 1) + "|"]
        for k, v in sorted(cs.items()):
            if k.startswith("torch:") or k.startswith("__amd"):
                continue   # input generation, not part of the layer
            lines.append(f"| {k} | " + " | ".join(f"{v[c]:.4g}" if c in v else "" for c in names) + " |")
        lines.append("")
        if fetch_f and write_f:
            lines += ["HBM traffic per dispatch (FETCH_SIZE and WRITE_SIZE, KiB, scaled by the calibration):", "",
                      "| kernel | fetch GB | write GB | total GB |", "|---|---|---|---|"]
            for k, v in sorted(cs.items()):
                if k.startswith("torch:") or k.startswith("__amd") or k == CALIB:
                    continue
                if "FETCH_SIZE" in v and "WRITE_SIZE" in v:
                    fb, wb = v["FETCH_SIZE"] * 1024 * fetch_f, v["WRITE_SIZE"] * 1024 * write_f
                    lines.append(f"| {k} | {fb / 1e9:.3f} | {wb / 1e9:.3f} | {(fb + wb) / 1e9:.3f} |")
            lines.append("")
        gu = next((v for k, v in cs.items() if k.startswith("gateup_kernel")), None)
        if gu and fetch_f and write_f and "FETCH_SIZE" in gu and "WRITE_SIZE" in gu:
            traffic = gu["FETCH_SIZE"] * 1024 * fetch_f + gu["WRITE_SIZE"] * 1024 * write_f
            lines += [f"gate/up HBM traffic per launch (scaled): fetch "
                      f"{gu['FETCH_SIZE'] * 1024 * fetch_f / 1e9:.3f} GB + write "
                      f"{gu['WRITE_SIZE'] * 1024 * write_f / 1e9:.3f} GB = {traffic / 1e9:.3f} GB", ""]
            # every layer kernel's bytes per launch, for the training bench's dominant kernel
            per_kernel = {k: v["FETCH_SIZE"] * 1024 * fetch_f + v["WRITE_SIZE"] * 1024 * write_f
                          for k, v in cs.items() if "FETCH_SIZE" in v and "WRITE_SIZE" in v and k != CALIB
                          and not k.startswith("torch:") and not k.startswith("__amd")}
            tf = os.path.join(args.out, "traffic_counters.json")
            table = json.load(open(tf)) if os.path.exists(tf) else {}
            train = args.workload.endswith("_train")
            table[args.workload] = {"gate_up_bytes_per_launch": traffic, "kernel_source_hash": source_hash(train),
                                    "fetch_scale": fetch_f, "write_scale": write_f,
                                    "gate_up_fetch_kib": gu["FETCH_SIZE"], "gate_up_write_kib": gu["WRITE_SIZE"],
                                    "bytes_per_launch": per_kernel}
            json.dump(table, open(tf, "w"), indent=1, sort_keys=True)
    out = os.path.join(args.out, args.name or f"rocprof_{args.workload}.md")
    open(out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _peaks(args):
    """Run the measured-ceiling probes and store their results."""
    import subprocess

    binary = os.path.join(ROOT, "mixture_experts_layer_deepseekmoe_amd", "peak_probes.bin")
    if not os.path.exists(binary):
        raise SystemExit(f"{binary} is missing: build first (python -m mixture_experts_layer_deepseekmoe_amd.build)")
    res = subprocess.run([binary], capture_output=True, text=True, check=True)
    probes = [json.loads(line) for line in res.stdout.splitlines() if line.startswith("{")]
    table = {p.pop("probe"): p for p in probes}
    os.makedirs(args.out, exist_ok=True)
    json.dump(table, open(os.path.join(args.out, "measured_peaks.json"), "w"), indent=1, sort_keys=True)
    print(json.dumps(table, indent=1, sort_keys=True))


def _library(args):
    """Time the vendor GEMM library (hipBLASLt, called through torch) on the
    workload's gate/up and down products, as a reference point for the
    grouped GEMMs: one dense GEMM over all grouped rows with a single weight
    matrix (the weight stays in cache), and a batched GEMM with one weight
    matrix per routed expert and T K / N_r rows each (every weight read from
    HBM, as in the layer, but uniform groups, no row gather and no shared
    expert).  bf16 only."""
    sys.path.insert(0, ROOT)
    import torch

    from moe_workloads import get_config

    cfg = get_config(args.workload)
    if cfg.w_dtype != "bf16":
        raise SystemExit("library reference: bf16 workloads only")
    dev = "cuda"
    g = torch.Generator(device=dev).manual_seed(0)

    def timeit(fn, reps=10):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s0.record()
        for _ in range(reps):
            fn()
        s1.record()
        torch.cuda.synchronize()
        return s0.elapsed_time(s1) / reps

    def randn(*shape, scale=1.0):
        return torch.randn(*shape, device=dev, dtype=torch.bfloat16, generator=g) * scale

    R = cfg.T * (cfg.top_k + cfg.n_shared)
    per = cfg.T * cfg.top_k // cfg.n_routed
    out = {}
    for name, n, k in (("gate_up", 2 * cfg.inter, cfg.d), ("down", cfg.d, cfg.inter)):
        x, w = randn(R, k), randn(n, k, scale=0.02)
        ms = timeit(lambda: torch.nn.functional.linear(x, w))
        out[f"{name}_dense"] = {"shape": [R, n, k], "ms": round(ms, 4), "tflops": round(2 * R * n * k / ms / 1e9, 1)}
        del x, w
        # the right operand [E][K][N] contiguous (no transposed view)
        xb, wb = randn(cfg.n_routed, per, k), randn(cfg.n_routed, k, n, scale=0.02)
        ms = timeit(lambda: torch.bmm(xb, wb))
        out[f"{name}_batched"] = {"shape": [cfg.n_routed, per, n, k], "ms": round(ms, 4),
                                  "tflops": round(2 * cfg.n_routed * per * n * k / ms / 1e9, 1)}
        del xb, wb
        torch.cuda.empty_cache()
    out["torch"] = torch.__version__
    out["command"] = f"python -m mixture_experts_layer_deepseekmoe_amd.profiling library --workload {cfg.name}"
    f = os.path.join(args.out, "library_reference.json")
    table = json.load(open(f)) if os.path.exists(f) else {}
    table[cfg.name] = out
    os.makedirs(args.out, exist_ok=True)
    json.dump(table, open(f, "w"), indent=1, sort_keys=True)
    print(json.dumps(out, indent=1, sort_keys=True))


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    r = sub.add_parser("run")
    r.add_argument("--workload", default="bf16_d7168")
    r.add_argument("--steps", type=int, default=3)
    r.add_argument("--train", action="store_true", help="training steps (moe_forward_train + moe_backward)")
    s = sub.add_parser("summarize")
    s.add_argument("--trace")
    s.add_argument("--pmc", nargs="*")
    s.add_argument("--workload", default="bf16_d7168")
    s.add_argument("--out", default=os.path.join(ROOT, "profiles"))
    s.add_argument("--name")
    s.add_argument("--command", nargs="*")
    pk = sub.add_parser("peaks")
    pk.add_argument("--out", default=os.path.join(ROOT, "profiles"))
    lb = sub.add_parser("library")
    lb.add_argument("--workload", default="bf16_d7168")
    lb.add_argument("--out", default=os.path.join(ROOT, "profiles"))
    args = ap.parse_args()
    {"run": _run, "summarize": _summarize, "peaks": _peaks, "library": _library}[args.cmd](args)


if __name__ == "__main__":
    main()
