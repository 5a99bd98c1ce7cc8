"""Benchmark of the MoE FFN layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config I]

A step is one pass of the whole hot path over one batch already resident in
HBM: router (logits + top-k), permute, expert gate/up + SwiGLU, expert down,
combine, each through its C-ABI entry point on torch's current stream, with a
HIP event after each so every stage is timed inside the timed region.  The
default workload is the Mixtral-8x7B-shaped decode layer (T=16, d=4096, 8
experts top-2, d_ff=14336, bf16).  Prints one JSON line.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0            # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0        # dense bf16 MFMA
PEAK_FP32_VALU_TFLOPS = 78.6     # 256 CU x 64 lanes x 2 flop x 2.4 GHz, no packed math
METRIC = "MoE-layer tokens/sec at 1 GPU; decode HBM GB/s and prefill TFLOP/s vs roofline"
STAGES = ["router", "permute", "gate_up", "down", "combine"]


def accounting(cfg, touched: int):
    """Algorithmic bytes and flops of each stage (each weight byte of a
    touched expert counted once; activations in and out once)."""
    T, k, N, d, f = cfg.T, cfg.top_k, cfg.n_experts, cfg.d_model, cfg.d_ff
    wb = {"f32": 4, "bf16": 2, "fp8": 1, "mxfp4": 0.5}[cfg.w_dtype]
    ab = 4 if cfg.act_dtype == "f32" else 2
    sh = cfg.n_shared
    rows = T * k + sh * T
    mats = touched + sh
    if cfg.w_dtype == "fp8":      # float32 per 128x128 block
        sc13, sc2 = 2 * (f // 128) * (d // 128) * 4, (f // 128) * (d // 128) * 4
    elif cfg.w_dtype == "mxfp4":  # one byte per 32 inputs
        sc13, sc2 = 2 * f * (d // 32), d * (f // 32)
    else:
        sc13 = sc2 = 0
    st = {
        "router": dict(bytes=T * d * ab + d * N * 4 + T * k * 8, flops=2 * T * d * N),
        "permute": dict(bytes=T * k * 4 + (2 * N + 1) * 4 + 2 * T * k * 4, flops=0),
        "gate_up": dict(bytes=int(mats * (2 * f * d * wb + sc13)) + rows * d * ab + rows * f * ab,
                        flops=2 * rows * d * 2 * f),
        "down": dict(bytes=int(mats * (d * f * wb + sc2)) + rows * f * ab + rows * d * ab,
                     flops=2 * rows * f * d),
        "combine": dict(bytes=rows * d * ab + T * d * ab + T * k * 8, flops=2 * T * k * d),
    }
    layer = dict(bytes=int(mats * (3 * f * d * wb + sc13 + sc2)) + d * N * 4 + 2 * T * d * ab,
                 flops=sum(v["flops"] for v in st.values()))
    return st, layer


def roofline_for(cfg, stage: dict, ms: float):
    flops, byts = stage["flops"], stage["bytes"]
    if cfg.w_dtype == "f32":
        peak_f = PEAK_FP32_VALU_TFLOPS
    else:
        peak_f = PEAK_BF16_TFLOPS
    ai = flops / max(byts, 1)
    ridge = peak_f * 1e12 / (PEAK_HBM_GBS * 1e9)
    if ai < ridge:
        ach = byts / (ms * 1e-3) / 1e9
        return {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(ach / PEAK_HBM_GBS, 4)}
    ach = flops / (ms * 1e-3) / 1e12
    bound = "alu" if cfg.w_dtype == "f32" else "mfma"
    return {"bound": bound, "achieved": round(ach, 1), "peak": peak_f, "unit": "TFLOP/s",
            "frac": round(ach / peak_f, 4)}


def measured_traffic(workload: str):
    """HBM bytes per launch of the gate/up kernel from the committed rocprofv3
    counter summary, or None when there is none for this workload or the
    kernel source has changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"traffic_{workload.replace('-', '_')}_T16.json")
    if workload != "mixtral-decode" or not os.path.exists(path):
        return None
    rec = json.load(open(path))
    src = open(os.path.join(ROOT, rec["source"]), "rb").read()
    if hashlib.sha256(src).hexdigest() != rec["source_sha256"]:
        return None
    return rec["traffic_bytes_per_launch"]


def achievable(torch):
    """Measured ceilings on this GPU beside the spec peaks: a plain device copy
    of 1 GiB (read + write bytes over its time) and a dense 8192^3 bf16
    matrix product (the vendor BLAS, contiguous operands)."""
    n = 1 << 30
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    a = torch.randn(8192, 8192, device="cuda").to(torch.bfloat16)
    b = torch.randn(8192, 8192, device="cuda").to(torch.bfloat16)
    out = {}
    for name, fn, work in (("hbm_copy_GBps", lambda: torch.mul(src, 1.0, out=dst), 2 * n / 1e9),
                           ("mfma_bf16_TFLOPs", lambda: torch.matmul(a, b), 2 * 8192 ** 3 / 1e12)):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            fn()
        e1.record()
        torch.cuda.synchronize()
        out[name] = round(work / (e0.elapsed_time(e1) / 10 * 1e-3), 1)
    del src, dst, a, b
    torch.cuda.empty_cache()
    return out


def cpu_baseline(cfg, x_cpu, n_tokens: int):
    """Time the CPU oracle (as it stands) on a bounded sample of the same
    workload: the first n_tokens tokens, weights decoded from their stored
    bits inside the timed region."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import oracle.moe_oracle as O
    from mixture_experts_ffn_09_amd import workloads as W
    from tests import _harness as Hh

    xs = x_cpu[:n_tokens]
    w_r, off, bias = Hh.oracle_router(cfg)
    R = O.route_tokens(Hh.x_f64(cfg, xs), w_r, cfg.top_k, cfg.route, off, bias)
    need = sorted(set(int(e) for e in R.idx.reshape(-1))) + ([cfg.n_experts] if cfg.n_shared else [])
    stored = {e: W.make_expert(cfg, e) for e in need}      # generation is not timed

    def expert(e):
        w = stored[e]
        return tuple(Hh.decode_weight(cfg, w, kk) for kk in ("gate", "up", "down"))

    # repeat the sample until about 10 s of CPU work have been timed
    reps, secs = 0, 0.0
    while reps == 0 or secs < CPU_SECONDS:
        t0 = time.perf_counter()
        xo = Hh.x_f64(cfg, xs)
        O.moe_forward(xo, w_r, expert, cfg.top_k, cfg.route, off, bias,
                      expert(cfg.n_experts) if cfg.n_shared else None)
        secs += time.perf_counter() - t0
        reps += 1
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    return {"value": round(n_tokens * reps / secs, 3), "unit": "tokens/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"first {n_tokens} of {cfg.T} tokens x {reps} runs, {len(need)} experts "
                      f"decoded from stored bits, float64 NumPy, {secs:.2f} s"}


CPU_SAMPLE = {0: 64, 1: 16, 2: 16, 3: 4, 4: 8, 5: 16}
CPU_SECONDS = 10.0


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=1, help="workload index (1 = Mixtral decode)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB, --steps times (calibrates "
                         "the HBM byte counters)")
    a = ap.parse_args()
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(expert- or token-parallel sharding is a design, not code)", file=sys.stderr)
        sys.exit(2)

    import torch

    if a.copy_probe:
        n = a.copy_probe << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(a.steps):
            torch.mul(src, 1.0, out=dst)   # reads n bytes, writes n bytes
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "launches": a.steps}))
        return

    from mixture_experts_ffn_09_amd import moe, workloads as W
    from mixture_experts_ffn_09_amd.layer import build_device_layer

    cfg = W.CONFIGS[a.config]
    print(f"[bench] building {cfg.name}", file=sys.stderr, flush=True)
    L = build_device_layer(cfg)
    x_cpu = W.make_x(cfg)
    x = x_cpu.to("cuda")
    T, k, N, d, f = cfg.T, cfg.top_k, cfg.n_experts, cfg.d_model, cfg.d_ff
    adt = x.dtype
    s = L.shape_for(T)
    ws = L.workspace()
    rb = L.routing_buffers()
    routing = moe.make_routing(**rb)
    h = torch.empty(T * k, f, dtype=adt, device="cuda")
    y = torch.empty(T * k, d, dtype=adt, device="cuda")
    h_sh = torch.empty(T, f, dtype=adt, device="cuda") if cfg.n_shared else None
    y_sh = torch.empty(T, d, dtype=adt, device="cuda") if cfg.n_shared else None
    out = torch.empty_like(x)

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        moe.moe_router_topk(s, x, L.weights, rb["topk_idx"], rb["topk_w"], ws)
        if ev is not None:
            ev[1].record()
        moe.moe_permute(s, rb["topk_idx"], None, routing, ws)
        if ev is not None:
            ev[2].record()
        moe.moe_expert_gate_up(s, x, None, rb["perm_token"], rb["offsets"], L.weights, h, h_sh, ws)
        if ev is not None:
            ev[3].record()
        moe.moe_expert_down(s, h, h_sh, rb["offsets"], L.weights, y, y_sh, ws)
        if ev is not None:
            ev[4].record()
        moe.moe_combine(s, y, y_sh, rb["inv_perm"], rb["topk_w"], out)
        if ev is not None:
            ev[5].record()

    def forward():
        moe.moe_layer_forward(s, L.weights, x, out, ws, routing)

    for _ in range(a.warmup):
        forward()
        step()
    torch.cuda.synchronize()

    # Timed region 1 (the reported value): K steps of the single C-ABI call
    # that runs the whole layer, nothing else on the stream.
    print(f"[bench] timing {a.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(a.steps):
        forward()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / a.steps

    # Timed region 2: the same work through the per-stage entry points, with
    # HIP events recorded on the launch stream between stages; these give
    # each stage's kernel time (the event records add a few microseconds to
    # the step, so this region's step time is reported only for reference).
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(a.steps)]
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    for i in range(a.steps):
        step(events[i])
    torch.cuda.synchronize()
    staged_ms = (time.perf_counter() - t2) * 1e3 / a.steps
    stage_ms = {name: sum(ev[j].elapsed_time(ev[j + 1]) for ev in events) / a.steps
                for j, name in enumerate(STAGES)}

    # Next-row kernels, timed on the same stream: load statistics of this
    # batch plus one selection-bias step (on a scratch copy of the bias)
    N_ = cfg.n_experts
    st_out = [torch.empty(N_, device="cuda"), torch.empty(N_, device="cuda"),
              torch.empty(1, device="cuda")]
    bias_scratch = (L.tensors["select_bias"].clone() if cfg.route == "sigmoid" else None)
    for _ in range(2):
        moe.moe_load_stats(s, x, L.weights, rb["counts"], ws, 0.01, 1e-3, *st_out, bias_scratch)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(a.steps):
        moe.moe_load_stats(s, x, L.weights, rb["counts"], ws, 0.01, 1e-3, *st_out, bias_scratch)
    e1.record()
    torch.cuda.synchronize()
    ls_ms = e0.elapsed_time(e1) / a.steps
    ls_bytes = T * d * (2 if adt == torch.bfloat16 else 4) + d * N_ * 4 + 4 * N_ * 4
    ls_gbs = ls_bytes / (ls_ms * 1e-3) / 1e9

    # Capacity-limited dispatch at capacity factor 1.0: the capped routing on
    # its own, and the whole layer with it
    cap = -(-T * k // N_)  # ceil(1.0 * T * k / N)
    rc = {kk: torch.empty_like(v) for kk, v in rb.items() if kk in
          ("counts", "offsets", "perm_token", "inv_perm")}
    rcs = moe.make_routing(**rc)
    out_c = torch.empty_like(x)
    for _ in range(2):
        moe.moe_permute_capacity(s, rb["topk_idx"], cap, rcs, ws)
        moe.moe_layer_forward_capacity(s, L.weights, x, out_c, cap, ws)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(a.steps):
        moe.moe_permute_capacity(s, rb["topk_idx"], cap, rcs, ws)
    e1.record()
    torch.cuda.synchronize()
    cap_ms = e0.elapsed_time(e1) / a.steps
    kept = int(rc["offsets"][N_].item())
    e0.record()
    for _ in range(a.steps):
        moe.moe_layer_forward_capacity(s, L.weights, x, out_c, cap, ws)
    e1.record()
    torch.cuda.synchronize()
    cap_layer_ms = e0.elapsed_time(e1) / a.steps

    # Group-limited selection, DeepSeek-V3 style: 8 groups of N/8 experts,
    # at most 4 groups per token (when the shape allows it)
    grouped = None
    if N_ % 8 == 0 and 4 * (N_ // 8) >= k:
        gi = torch.empty_like(rb["topk_idx"])
        gw_ = torch.empty_like(rb["topk_w"])
        for _ in range(2):
            moe.moe_router_topk_grouped(s, x, L.weights, 8, 4, gi, gw_, ws)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(a.steps):
            moe.moe_router_topk_grouped(s, x, L.weights, 8, 4, gi, gw_, ws)
        e1.record()
        torch.cuda.synchronize()
        g_router_ms = e0.elapsed_time(e1) / a.steps
        e0.record()
        for _ in range(a.steps):
            moe.moe_layer_forward_grouped(s, L.weights, x, out_c, 8, 4, ws)
        e1.record()
        torch.cuda.synchronize()
        g_layer_ms = e0.elapsed_time(e1) / a.steps
        grouped = {"n_groups": 8, "max_groups": 4, "router_topk_ms": round(g_router_ms, 4),
                   "layer_ms": round(g_layer_ms, 4),
                   "layer_tokens_per_s": round(T / (g_layer_ms * 1e-3), 2),
                   "what": "moe_router_topk_grouped and moe_layer_forward_grouped"}

    counts = rb["counts"].cpu()
    touched = int((counts > 0).sum())
    st, layer = accounting(cfg, touched)
    stages = {}
    for name in STAGES:
        r = roofline_for(cfg, st[name], stage_ms[name])
        stages[name] = {"ms": round(stage_ms[name], 4), "bytes": st[name]["bytes"],
                        "flops": st[name]["flops"], "bound": r["bound"], "frac": r["frac"],
                        "achieved": r["achieved"], "unit": r["unit"]}
    dom = "gate_up"
    roof = roofline_for(cfg, st[dom], stage_ms[dom])
    roof["traffic"] = measured_traffic(cfg.name)
    roof["kernel"] = "expert gate/up + SwiGLU (moe_expert_gate_up)"
    ach = achievable(torch)
    ach_peak = ach["hbm_copy_GBps"] if roof["bound"] == "hbm" else ach["mfma_bf16_TFLOPs"]
    if roof["bound"] in ("hbm", "mfma"):
        ach["dominant_kernel_frac_of_achievable"] = round(roof["achieved"] / ach_peak, 4)
    layer_gbs = layer["bytes"] / (ms_step * 1e-3) / 1e9
    layer_tflops = layer["flops"] / (ms_step * 1e-3) / 1e12

    rec = {
        "metric": METRIC, "value": round(T / (ms_step * 1e-3), 2), "unit": "tokens/s",
        "n_gpus": 1, "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": {"f32": "f32", "bf16": "bf16", "fp8": "fp8-e4m3 weights, bf16 activations",
                  "mxfp4": "mxfp4 (e2m1 + e8m0) weights, bf16 activations"}[cfg.w_dtype],
        "data": "synthetic (seeded random weights and inputs)",
        "config": {"workload": cfg.name, "T": T, "d_model": d, "n_experts": N, "top_k": k,
                   "d_ff": f, "n_shared": cfg.n_shared, "route": cfg.route,
                   "weights": cfg.w_dtype, "experts_touched": touched,
                   "max_over_mean_load": round(float(counts.max()) / max(1e-9, float(counts.float().mean())), 3)},
        "roofline": roof,
        "achievable": ach,
        "layer": {"algorithmic_bytes": layer["bytes"], "flops": layer["flops"],
                  "hbm_GBps": round(layer_gbs, 1), "hbm_frac": round(layer_gbs / PEAK_HBM_GBS, 4),
                  "TFLOPs": round(layer_tflops, 2),
                  "staged_ms_per_step": round(staged_ms, 4)},
        "stages": stages,
        "next_rows": {"load_stats": {
            "ms": round(ls_ms, 4), "bytes": ls_bytes, "bound": "hbm",
            "achieved": round(ls_gbs, 1), "unit": "GB/s", "frac": round(ls_gbs / PEAK_HBM_GBS, 4),
            "what": "moe_load_stats: router probabilities, shares, balancing term, bias step"},
            "capacity_dispatch": {
                "capacity_factor": 1.0, "capacity": cap, "kept": kept, "assignments": T * k,
                "permute_capacity_ms": round(cap_ms, 4), "layer_ms": round(cap_layer_ms, 4),
                "layer_tokens_per_s": round(T / (cap_layer_ms * 1e-3), 2),
                "what": "moe_permute_capacity and moe_layer_forward_capacity, C = ceil(T*k/N)"},
            "group_limited": grouped},
    }
    if not a.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = cpu_baseline(cfg, x_cpu, min(T, CPU_SAMPLE.get(a.config, 8)))
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
