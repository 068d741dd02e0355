#!/usr/bin/env python3
"""Throughput of the DeepSeekMoE layer on one MI355X.

One step = one pass of the whole hot path over one batch: moe_forward (router
GEMM + top-K + gates, expert grouping, grouped gate/up GEMM with SwiGLU,
grouped down GEMM, combine) followed by the aux-loss-free bias update from the
step's expert counts.  Inputs are seeded synthetic tensors resident in HBM
before timing starts.  Prints ONE JSON line on stdout.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload bf16_d7168]
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/sec + grouped-GEMM % MFMA peak, d=7168 N_r=256 K=8, 1 GPU"
PEAK_TFLOPS = {"bf16": 2500.0, "e4m3": 5000.0, "f32": 157.3}
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def measured_traffic(workload: str, kernel: str = "gateup_kernel", train: bool = False):
    """HBM bytes per launch of ``kernel`` (default: the gate/up GEMM) from the
    committed rocprofv3 counter runs (record ``workload``, or ``workload``_train),
    if they were taken on the current GEMM sources; else None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    table = json.load(open(TRAFFIC_FILE))
    rec = table.get(workload + ("_train" if train else ""))
    from mixture_experts_layer_deepseekmoe_amd.profiling import source_hash
    if not rec or rec.get("kernel_source_hash") != source_hash(train):
        return None
    if kernel == "gateup_kernel" and not train:
        return rec.get("gate_up_bytes_per_launch")
    return next((v for k, v in rec.get("bytes_per_launch", {}).items() if k == kernel or k.startswith(kernel + "<")),
                None)


def measured_peaks():
    """Ceilings measured on this chip by profiling.py peaks (MFMA with random
    operands, HBM read stream), if stored; else None."""
    f = os.path.join(os.path.dirname(TRAFFIC_FILE), "measured_peaks.json")
    return json.load(open(f)) if os.path.exists(f) else None


def library_reference(workload):
    """hipBLASLt timings of GEMMs of the workload's sizes (profiling.py
    library), if stored; else None."""
    f = os.path.join(os.path.dirname(TRAFFIC_FILE), "library_reference.json")
    return json.load(open(f)).get(workload) if os.path.exists(f) else None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="bf16_d7168")
    ap.add_argument("--cpu-sample-tokens", type=int, default=256)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--train", action="store_true",
                    help="time the training step instead: moe_forward_train + moe_backward (bf16)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (expert and data sharding are "
              "designed, not implemented); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import mixture_experts_layer_deepseekmoe_amd as moe
    from mixture_experts_layer_deepseekmoe_amd.binding import HipEvents
    from moe_workloads import get_config, make_inputs

    cfg = get_config(args.workload)
    torch.cuda.set_device(0)
    if args.train:
        return train_bench(args, cfg)
    log(f"[bench] workload {cfg.name}: generating seeded inputs")
    inp = make_inputs(cfg, 0, weights_device="cuda")
    shape = moe.LayerShape.from_config(cfg)
    u = inp.u.cuda().contiguous()
    cen = inp.centroids.cuda().contiguous()
    bias = inp.bias.cuda().contiguous()
    weights = moe.prepare_weights(cfg, inp)
    ws = moe.alloc_workspace(shape)
    routing = moe.alloc_routing(shape)
    y = torch.empty((cfg.T, cfg.d), dtype=torch.float32 if cfg.out_dtype == "f32" else torch.bfloat16,
                    device="cuda")
    TK = cfg.T * cfg.top_k
    torch.cuda.synchronize()

    def step(trace=None):
        moe.moe_forward(shape, u, cen, bias, weights, y=y, routing=routing, workspace=ws, trace=trace)
        moe.moe_update_bias(bias, routing["expert_counts"], TK, 0.001)

    log(f"[bench] warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # The timed steps record events around the dominant kernel only (its
    # launches, timed on the library's stream, give the roofline); the other
    # stages are timed on a few further steps, so that their events do not
    # sit inside the timed region.
    events = [HipEvents(("gate_up",)) for _ in range(args.steps)]
    log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(events[k].trace)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    elapsed = t1 - t0
    gate_up_ms = sum(ev.elapsed_ms()["gate_up"] for ev in events) / args.steps
    for ev in events:
        ev.close()
    n_diag = min(args.steps, 10)
    diag = [HipEvents() for _ in range(n_diag)]
    for k in range(n_diag):
        step(diag[k].trace)
    torch.cuda.synchronize()
    stages = {}
    for ev in diag:
        for name, ms in ev.elapsed_ms().items():
            stages[name] = stages.get(name, 0.0) + ms / n_diag
    for ev in diag:
        ev.close()
    stages["gate_up"] = gate_up_ms
    counts = routing["expert_counts"].cpu().numpy()
    log(f"[bench] {elapsed / args.steps * 1e3:.3f} ms/step; stages (ms): "
        + ", ".join(f"{k} {v:.4f}" for k, v in stages.items()))

    # ---------------- roofline of the dominant kernel (grouped gate/up GEMM)
    rows = TK + cfg.n_shared * cfg.T
    es = {"bf16": 2, "e4m3": 1, "f32": 4}[cfg.w_dtype]
    gu_flops = 2.0 * rows * 2 * cfg.inter * cfg.d
    dn_flops = 2.0 * rows * cfg.d * cfg.inter
    gu_s = stages["gate_up"] * 1e-3
    dn_s = stages["down"] * 1e-3
    peak = PEAK_TFLOPS[cfg.w_dtype]
    gu_tflops = gu_flops / gu_s / 1e12
    touched = int((counts > 0).sum())
    gu_bytes = (touched + cfg.n_shared) * 2 * cfg.inter * cfg.d * es + cfg.T * cfg.d * es + rows * cfg.inter * es
    # The binding roof follows the kernel's arithmetic intensity: below the
    # ridge (peak flops / HBM bandwidth) the weight stream bounds it.
    intensity = gu_flops / gu_bytes
    ridge = peak * 1e12 / (PEAK_HBM_GBS * 1e9)
    gu_gbs = gu_bytes / gu_s / 1e9
    if intensity < ridge:
        bound, achieved, peak_r, unit = "hbm", gu_gbs, PEAK_HBM_GBS, "GB/s"
    else:
        bound, achieved, peak_r, unit = "mfma", gu_tflops, peak, "TFLOP/s"
    roofline = {"bound": bound, "kernel": "gateup_kernel (grouped gate/up GEMM + SwiGLU)",
                "achieved": round(achieved, 2), "peak": peak_r, "unit": unit,
                "frac": round(achieved / peak_r, 4), "traffic": measured_traffic(cfg.name),
                "flops_per_launch": gu_flops, "algorithmic_bytes_per_launch": gu_bytes,
                "flop_per_byte": round(intensity, 1), "ridge_flop_per_byte": round(ridge, 1),
                "mfma_tflops": round(gu_tflops, 2), "mfma_frac": round(gu_tflops / peak, 4),
                "hbm_gbs": round(gu_gbs, 1), "hbm_frac": round(gu_gbs / PEAK_HBM_GBS, 4),
                "avg_launch_ms": round(stages["gate_up"], 4)}
    mp = measured_peaks()
    if mp:
        key = "mfma_e4m3_16x16x128_random_operands" if cfg.w_dtype == "e4m3" else "mfma_bf16_16x16x32_random_operands"
        m_tf = mp.get(key, {}).get("tflops_sustained")
        m_bw = mp.get("hbm_read_lds_dma_paired_64B", {}).get("gbs_best")
        if m_tf and m_bw and cfg.w_dtype != "f32":
            roofline["measured_ceilings"] = {
                "mfma_tflops_random_operands": m_tf, "mfma_frac": round(gu_tflops / m_tf, 4),
                "hbm_read_gbs": m_bw, "hbm_frac": round(gu_gbs / m_bw, 4)}
    lib = library_reference(cfg.name)
    if lib and "gate_up_batched" in lib:
        # the vendor library on the same products: uniform batches (one weight
        # per expert, T K / N_r rows each) and one dense GEMM with a single weight
        dn_tflops = dn_flops / dn_s / 1e12
        roofline["library_reference"] = {
            "batched_tflops": lib["gate_up_batched"]["tflops"], "dense_tflops": lib["gate_up_dense"]["tflops"],
            "vs_batched": round(gu_tflops / lib["gate_up_batched"]["tflops"], 4),
            "vs_dense": round(gu_tflops / lib["gate_up_dense"]["tflops"], 4),
            "down_vs_batched": round(dn_tflops / lib["down_batched"]["tflops"], 4),
            "down_vs_dense": round(dn_tflops / lib["down_dense"]["tflops"], 4)}
    grouped_frac = (gu_flops + dn_flops) / (gu_s + dn_s) / 1e12 / peak

    xs = 4 if cfg.x_dtype == "f32" else 2
    os_ = 4 if cfg.out_dtype == "f32" else 2
    ys = 4 if cfg.w_dtype == "f32" else 2
    hbm = {
        "route": (cfg.T * cfg.d * xs + cfg.n_routed * cfg.d * xs + TK * 8) / (stages["route"] * 1e-3) / 1e9,
        "group": (TK * 4 * 3 + TK * 8) / (stages["group"] * 1e-3) / 1e9,
        "combine": (cfg.T * cfg.d * xs + rows * cfg.d * ys + cfg.T * cfg.d * os_ + TK * 8)
                   / (stages["combine"] * 1e-3) / 1e9,
    }

    result = {
        "metric": METRIC,
        "value": round(cfg.T * args.steps / elapsed, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.w_dtype,
        "data": "synthetic (seeded N(0,1) activations, N(0,0.006) weights, N(0,0.02) centroids, random init)",
        "config": {"workload": cfg.name, "T": cfg.T, "d": cfg.d, "n_routed": cfg.n_routed,
                   "n_shared": cfg.n_shared, "inter": cfg.inter, "top_k": cfg.top_k,
                   "x_dtype": cfg.x_dtype, "w_dtype": cfg.w_dtype, "out_dtype": cfg.out_dtype,
                   "parallelism": "single GPU"},
        "roofline": roofline,
        "grouped_gemm_mfma_frac": round(grouped_frac, 4),
        "stage_ms": {k: round(v, 4) for k, v in stages.items()},
        "stage_ms_source": f"gate_up: events over the {args.steps} timed steps; others: {n_diag} traced steps after them",
        "stage_hbm_frac": {k: round(v / PEAK_HBM_GBS, 4) for k, v in hbm.items()},
        "load": {"max_over_mean": round(float(counts.max() / counts.mean()), 3), "experts_touched": touched},
    }

    if cfg.zipf_s is not None:
        result["bias_loop"] = bias_loop(cfg, shape, u, cen, ws)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(cfg, inp, args.cpu_sample_tokens, result)
    print(json.dumps(result), flush=True)


def train_bench(args, cfg):
    """The training step on one GPU: moe_forward_train, then moe_backward for
    a seeded N(0, 1) upstream gradient.  Prints one JSON line; the roofline is
    that of the slowest backward GEMM (events over the timed steps, on the
    library's stream)."""
    import torch

    import mixture_experts_layer_deepseekmoe_amd as moe
    from mixture_experts_layer_deepseekmoe_amd.binding import BACKWARD_STAGES, HipEvents
    from moe_workloads import make_inputs

    if cfg.x_dtype != "bf16" or cfg.w_dtype not in ("bf16", "e4m3"):
        print("the training path takes bf16 activations with bf16 or e4m3 weights", file=sys.stderr)
        sys.exit(2)
    fp8 = cfg.w_dtype == "e4m3"
    log(f"[bench] train workload {cfg.name}: generating seeded inputs")
    inp = make_inputs(cfg, 0, weights_device="cuda")
    shape = moe.LayerShape.from_config(cfg)
    u, cen, bias = (t.cuda().contiguous() for t in (inp.u, inp.centroids, inp.bias))
    weights = moe.prepare_weights(cfg, inp, train=True)
    ws = moe.alloc_train_workspace(shape)
    grads = moe.alloc_weight_grads(shape)
    y = torch.empty((cfg.T, cfg.d), dtype=torch.float32 if cfg.out_dtype == "f32" else torch.bfloat16, device="cuda")
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    dy = torch.randn((cfg.T, cfg.d), generator=g, device="cuda", dtype=torch.float32)
    TK = cfg.T * cfg.top_k
    torch.cuda.synchronize()

    def step(trace_b=None):
        moe.moe_forward_train(shape, u, cen, bias, weights, ws, y=y)
        moe.moe_backward(shape, u, cen, weights, dy, ws, grads=grads, trace=trace_b)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [HipEvents(BACKWARD_STAGES) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(events[k].trace)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    stages = {}
    for ev in events:
        for name, ms in ev.elapsed_ms().items():
            stages[name] = stages.get(name, 0.0) + ms / args.steps
        ev.close()
    fw = HipEvents()
    moe.moe_forward_train(shape, u, cen, bias, weights, ws, y=y, trace=fw.trace)
    torch.cuda.synchronize()
    stages.update({"fwd_" + k: v for k, v in fw.elapsed_ms().items()})
    fw.close()
    log(f"[bench] train {elapsed / args.steps * 1e3:.3f} ms/step; stages (ms): "
        + ", ".join(f"{k} {v:.4f}" for k, v in stages.items()))

    R = TK + cfg.n_shared * cfg.T
    d, I = cfg.d, cfg.inter
    G = cfg.n_routed + cfg.n_shared
    routing = moe.moe_route(shape, u, cen, bias)
    counts = routing["expert_counts"].cpu().numpy()
    touched = int((counts > 0).sum()) + cfg.n_shared
    # algorithmic flops and bytes per launch of each backward GEMM (operands
    # of e bytes: 2 bf16, 1 e4m3; bf16 Dgrad outputs, fp32 weight gradients);
    # an FP8 stage also quantises its operands (timed with it, not counted)
    e = 1 if fp8 else 2
    gemms = {
        "bwd_dgrad_down": (2.0 * R * d * I, touched * d * I * e + R * d * e + 2 * R * 2 * I * 2 + R * I * 2),
        "bwd_dgrad_gate_up": (2.0 * R * 2 * I * d, touched * 2 * I * d * e + R * 2 * I * e + R * d * 2),
        "bwd_wgrad_down": (2.0 * R * d * I, R * d * e + R * I * e + G * d * I * 4),
        "bwd_wgrad_gate_up": (2.0 * R * 2 * I * d, R * 2 * I * e + R * d * e + G * 2 * I * d * 4),
    }
    peak_tf = PEAK_TFLOPS["e4m3" if fp8 else "bf16"]
    lines = {}
    for name, (fl, by) in gemms.items():
        sec = stages[name] * 1e-3
        tf, gbs = fl / sec / 1e12, by / sec / 1e9
        ridge = peak_tf * 1e12 / (PEAK_HBM_GBS * 1e9)
        if fl / by < ridge:
            bound, ach, pk, unit = "hbm", gbs, PEAK_HBM_GBS, "GB/s"
        else:
            bound, ach, pk, unit = "mfma", tf, peak_tf, "TFLOP/s"
        lines[name] = {"bound": bound, "achieved": round(ach, 2), "peak": pk, "unit": unit, "frac": round(ach / pk, 4),
                       "flops_per_launch": fl, "algorithmic_bytes_per_launch": by, "avg_launch_ms": round(stages[name], 4),
                       "mfma_frac": round(tf / peak_tf, 4), "hbm_frac": round(gbs / PEAK_HBM_GBS, 4)}
    dominant = max(gemms, key=lambda k: stages[k])
    # the dominant stage's GEMM kernel (the FP8 Dgrad runs on the forward's down kernel, not told apart)
    kern = {"bwd_wgrad_gate_up": "wgrad8_gateup_kernel" if fp8 else "wgrad_gateup_kernel",
            "bwd_wgrad_down": "wgrad8_down_kernel" if fp8 else "wgrad_down_kernel",
            "bwd_dgrad_gate_up": None if fp8 else "dgrad_gateup_kernel",
            "bwd_dgrad_down": None if fp8 else "dgrad_down_kernel"}[dominant]
    roofline = dict(lines[dominant], kernel=dominant,
                    traffic=measured_traffic(cfg.name, kern, train=True) if kern else None)
    result = {
        "metric": f"MoE-layer training step tokens/sec (forward + backward, {'fp8' if fp8 else 'bf16'}), "
                  f"d={d} N_r={cfg.n_routed} K={cfg.top_k}, 1 GPU",
        "value": round(cfg.T * args.steps / elapsed, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(elapsed / args.steps * 1e3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "e4m3" if fp8 else "bf16",
        "data": "synthetic (seeded N(0,1) activations and upstream gradient, N(0,0.006) weights, random init)",
        "config": {"workload": cfg.name, "T": cfg.T, "d": d, "n_routed": cfg.n_routed, "n_shared": cfg.n_shared,
                   "inter": I, "top_k": cfg.top_k, "parallelism": "single GPU", "step": "forward_train + backward"},
        "roofline": roofline, "backward_gemms": lines, "stage_ms": {k: round(v, 4) for k, v in stages.items()},
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = train_cpu_baseline(cfg, inp, dy, 32)
    print(json.dumps(result), flush=True)


def train_cpu_baseline(cfg, inp, dy, n_tokens):
    """The CPU oracle's forward + backward on the first n_tokens tokens."""
    import threadpoolctl

    from moe_workloads import to_numpy_f32
    from oracle import moe_oracle as O

    n = min(n_tokens, cfg.T)
    u, E, b = to_numpy_f32(inp.u[:n]), to_numpy_f32(inp.centroids), inp.bias.numpy()
    routed = lambda e: (to_numpy_f32(inp.w_gate_up[e]), to_numpy_f32(inp.w_down[e]))
    shared = [(to_numpy_f32(inp.ws_gate_up[s]), to_numpy_f32(inp.ws_down[s])) for s in range(cfg.n_shared)]
    host_cores = len(os.sched_getaffinity(0))
    cap = int(os.environ.get("OMP_NUM_THREADS", "0") or 0)
    threads = min(host_cores, cap) if cap > 0 else host_cores
    dyn = dy[:n].cpu().numpy()
    with threadpoolctl.threadpool_limits(limits=threads):
        used = max([p.get("num_threads", 1) for p in threadpoolctl.threadpool_info()], default=1)
        t0 = time.perf_counter()
        O.layer_backward(u, E, b, cfg.top_k, routed, cfg.n_routed, shared, dyn, fp8=cfg.w_dtype == "e4m3")
        dt = time.perf_counter() - t0
    return {"value": round(n / dt, 3), "unit": "tokens/s", "cores": used, "kind": "oracle",
            "host_cores_visible": host_cores,
            "sample": f"first {n} of the {cfg.T} tokens, fp64 forward + backward with every weight gradient"
                      + (" (FP8 quantisation steps included)" if cfg.w_dtype == "e4m3" else ""),
            "seconds": round(dt, 2)}


def bias_loop(cfg, shape, u, cen, ws, steps=100):
    """The skewed batch's aux-loss-free balancing loop: from b = 0, each step
    routes the same batch (moe_route) and updates the bias from its expert
    counts (moe_update_bias, gamma = 0.001); reports max/mean expert load per
    step (before that step's update)."""
    import torch

    import mixture_experts_layer_deepseekmoe_amd as moe

    b = torch.zeros(cfg.n_routed, dtype=torch.float32, device="cuda")
    routing = moe.alloc_routing(shape)
    TK = cfg.T * cfg.top_k
    ratios = []
    for _ in range(steps):
        moe.moe_route(shape, u, cen, b, out=routing, workspace=ws)
        moe.moe_update_bias(b, routing["expert_counts"], TK, 0.001)
        c = routing["expert_counts"].cpu().numpy()
        ratios.append(round(float(c.max() / c.mean()), 3))
    log(f"[bench] bias loop: max/mean load {ratios[0]} -> {ratios[-1]} over {steps} steps")
    return {"steps": steps, "gamma": 0.001, "b0": 0.0, "load_max_over_mean_per_step": ratios}


def cpu_baseline(cfg, inp, n_tokens, result):
    """The CPU oracle, as it stands, on the first n_tokens tokens of the batch."""
    import numpy as np
    import threadpoolctl

    from moe_workloads import to_numpy_f32
    from oracle import moe_oracle as O

    n = min(n_tokens, cfg.T)
    u = to_numpy_f32(inp.u[:n])
    E = to_numpy_f32(inp.centroids)
    b = inp.bias.numpy()
    routed = lambda e: (to_numpy_f32(inp.w_gate_up[e]), to_numpy_f32(inp.w_down[e]))
    shared = [(to_numpy_f32(inp.ws_gate_up[s]), to_numpy_f32(inp.ws_down[s])) for s in range(cfg.n_shared)]
    # The BLAS pool gets one thread per host core this process may use,
    # capped by OMP_NUM_THREADS where the host sets one (the CPU share of
    # one GPU on a shared node).
    host_cores = len(os.sched_getaffinity(0))
    cap = int(os.environ.get("OMP_NUM_THREADS", "0") or 0)
    threads = min(host_cores, cap) if cap > 0 else host_cores
    with threadpoolctl.threadpool_limits(limits=threads):
        used = max([p.get("num_threads", 1) for p in threadpoolctl.threadpool_info()], default=1)
        log(f"[bench] cpu baseline: oracle on {n} tokens, {used} BLAS threads ({host_cores} host cores visible)")
        t0 = time.perf_counter()
        O.layer_forward(u, E, b, cfg.top_k, routed, cfg.n_routed, shared, fp8=cfg.fp8)
        dt = time.perf_counter() - t0
    return {"value": round(n / dt, 3), "unit": "tokens/s", "cores": used, "kind": "oracle",
            "host_cores_visible": host_cores, "omp_num_threads": cap or None,
            "sample": f"first {n} of the {cfg.T} tokens of the same seeded batch, full layer (fp64 NumPy; "
                      f"expert weights streamed from HBM per expert inside the timed region)",
            "seconds": round(dt, 2)}


if __name__ == "__main__":
    main()
