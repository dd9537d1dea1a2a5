#!/usr/bin/env python3
"""Benchmark of the gfx950 GEMM library on one MI355X.

Default workload (one "step"): the four bf16 GEMMs of a Llama-70B-like
transformer layer at M = 4096 tokens -- QKV 4096x10240x8192, O 4096x8192x8192,
gate/up 4096x57344x8192, down 4096x8192x28672 -- with A ~ N(0,1) RowMajor,
weights ~ N(0, 0.02^2) stored [N, K] (ColumnMajor B), fp32 accumulation, bf16 D.
Inputs are resident in HBM before the timed region starts.

Prints ONE JSON line: whole-step TFLOP/s, the roofline object of the dominant
kernel (per-launch durations from HIP events recorded on the launch stream
inside the timed region) and the CPU oracle's throughput on a bounded sample
(``cpu_baseline``). ``--workload`` selects the other workloads of the suite.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"bf16": 2516.6, "f16": 2516.6, "f8e4m3": 5033.2, "f32": 157.3}
PEAK_HBM_GBS = 8000.0
METRIC = "GEMM TFLOP/s and % of MI355X MFMA peak per dtype, 1 GPU"

WORKLOADS = ("layer", "down", "fp16_1024_relu", "grouped64", "fp8_decode", "fp32_small",
             "mx_layer", "layer_residual", "batched16", "layer_nn")


def source_hash() -> str:
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "dense_gemm_epilogue_02_amd", "csrc", "*"))):
        with open(f, "rb") as fh:
            h.update(os.path.basename(f).encode())
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when the kernels changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        t = json.load(fh)
    if t.get("source_hash") != source_hash():
        return None
    return t.get("hbm_bytes_per_launch")


# ----------------------------------------------------------------- workloads

def build_layer(names, lb="col"):
    import torch
    import synthetic as syn
    import dense_gemm_epilogue_02_amd as g
    dev = torch.device("cuda:0")
    plan = g.Plan("bf16", la="row", lb=lb, lc="row")
    items = []
    for i, name in enumerate(names):
        p = syn.config4(name, seed=i, lb=lb)
        A, B = p.A.to(dev), p.B.to(dev)
        D = torch.empty((p.M, p.N), dtype=torch.bfloat16, device=dev)
        items.append(dict(name=name, p=p, flops=p.flops, plan=plan,
                          call=(lambda A=A, B=B, D=D, p=p: plan.run(A, B, None, D, p.M, p.N, p.K,
                                                                     1.0, 0.0)),
                          bytes=p.M * p.K * 2 + p.K * p.N * 2 + p.M * p.N * 2,
                          describe=plan.describe(p.M, p.N, p.K)))
        del p.A, p.B
    return items, "bf16"


def build_fp16_relu():
    import torch
    import synthetic as syn
    import dense_gemm_epilogue_02_amd as g
    dev = torch.device("cuda:0")
    p = syn.config2()
    plan = g.Plan("f16", la="row", lb="row", lc="row", relu=True)
    A, B, C = p.A.to(dev), p.B.to(dev), p.C.to(dev)
    D = torch.empty_like(C)
    return [dict(name="fp16_1024_relu", p=p, flops=p.flops, plan=plan,
                 call=lambda: plan.run(A, B, C, D, p.M, p.N, p.K, 1.0, 1.0),
                 tune=lambda: plan.profile(A, B, C, D, p.M, p.N, p.K, 1.0, 1.0, iters=20),
                 bytes=3 * 1024 * 1024 * 2 + 1024 * 1024 * 2,
                 describe=plan.describe(p.M, p.N, p.K))], "f16"


def build_grouped():
    import torch
    import synthetic as syn
    import dense_gemm_epilogue_02_amd as g
    dev = torch.device("cuda:0")
    probs = syn.config3()
    plan = g.Plan("f16", la="row", lb="row", lc="row")
    args, flops, nbytes = [], 0, 0
    for p in probs:
        A, B = p.A.to(dev), p.B.to(dev)
        D = torch.empty((p.M, p.N), dtype=torch.float16, device=dev)
        args.append((p.M, p.N, p.K, A, B, None, D))
        flops += p.flops
        nbytes += 2 * (p.M * p.K + p.K * p.N + p.M * p.N)
    return [dict(name="grouped64", p=probs[0], flops=flops, plan=plan,
                 call=lambda: plan.run_grouped(args, 1.0, 0.0), bytes=nbytes,
                 describe={"kernel": "grouped", "tile": "128x128", "problems": len(probs)})], "f16"


def build_fp8():
    import torch
    import synthetic as syn
    import dense_gemm_epilogue_02_amd as g
    dev = torch.device("cuda:0")
    plan = g.Plan("f8e4m3", la="row", lb="col", lc="row")
    items = []
    for M in syn.DECODE_MS:
        for (N, K) in syn.DECODE_NK:
            p = syn.config5(M, N, K)
            A, B = p.A.to(dev), p.B.to(dev)
            sa = torch.tensor([p.scale_a], dtype=torch.float32, device=dev)
            sb = torch.tensor([p.scale_b], dtype=torch.float32, device=dev)
            D = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            items.append(dict(name=f"fp8_{M}x{N}x{K}", p=p, flops=p.flops, plan=plan,
                              call=(lambda A=A, B=B, D=D, sa=sa, sb=sb, p=p:
                                    plan.run(A, B, None, D, p.M, p.N, p.K, 1.0, 0.0, sa, sb)),
                              tune=(lambda A=A, B=B, D=D, p=p:
                                    plan.profile(A, B, None, D, p.M, p.N, p.K, 1.0, 0.0,
                                                 iters=10)),
                              bytes=M * K + K * N + M * N * 2,
                              describe=plan.describe(M, N, K)))
    return items, "f8e4m3"


def build_fp32():
    import torch
    import synthetic as syn
    import dense_gemm_epilogue_02_amd as g
    dev = torch.device("cuda:0")
    p = syn.config1()
    plan = g.Plan("f32", la="row", lb="row", lc="row")
    A, B, C = p.A.to(dev), p.B.to(dev), p.C.to(dev)
    D = torch.empty_like(C)
    return [dict(name="fp32_128x64x256", p=p, flops=p.flops, plan=plan,
                 call=lambda: plan.run(A, B, C, D, p.M, p.N, p.K, 1.0, 1.0),
                 tune=lambda: plan.profile(A, B, C, D, p.M, p.N, p.K, 1.0, 1.0, iters=50),
                 bytes=4 * (128 * 256 + 256 * 64 + 2 * 128 * 64),
                 describe=plan.describe(p.M, p.N, p.K))], "f32"


def build_mx_layer():
    """The four layer GEMMs in MXFP8 (e4m3 elements, E8M0 scales per 32 K)."""
    import torch
    import synthetic as syn
    import dense_gemm_epilogue_02_amd as g
    dev = torch.device("cuda:0")
    plan = g.Plan("f8e4m3", la="row", lb="col", lc="row")
    items = []
    for i, name in enumerate(("qkv", "o", "gate_up", "down")):
        M, N, K, A, B, xa, xb = syn.mx_layer_device(name, dev, seed=i)
        D = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        shape = type("S", (), dict(M=M, N=N, K=K))
        items.append(dict(name=name, p=shape, flops=2 * M * N * K, plan=plan,
                          call=(lambda A=A, B=B, D=D, xa=xa, xb=xb, M=M, N=N, K=K:
                                plan.run_mx(A, B, None, D, M, N, K, xa, xb)),
                          bytes=M * K + K * N + M * N * 2 + (M + N) * (K // 32),
                          describe=plan.describe(M, N, K)))
    torch.cuda.synchronize()
    return items, "f8e4m3"


def build_layer_residual():
    """O and down projections with the residual add fused as an auxiliary
    tensor (D = A W + X, X the M x N residual stream, bf16)."""
    import torch
    import synthetic as syn
    import dense_gemm_epilogue_02_amd as g
    dev = torch.device("cuda:0")
    plan = g.Plan("bf16", la="row", lb="col", lc="row")
    items = []
    for i, name in enumerate(("o", "down")):
        p = syn.config4(name, seed=i)
        A, B = p.A.to(dev), p.B.to(dev)
        gen = torch.Generator(device=dev)
        gen.manual_seed(100 + i)
        X = torch.randn((p.M, p.N), generator=gen, device=dev).to(torch.bfloat16)
        D = torch.empty((p.M, p.N), dtype=torch.bfloat16, device=dev)
        items.append(dict(name=name + "_residual", p=p, flops=p.flops, plan=plan,
                          call=(lambda A=A, B=B, D=D, X=X, p=p:
                                plan.run_aux(A, B, None, D, p.M, p.N, p.K, aux=X,
                                             aux_op="add", aux_pos="before")),
                          bytes=p.M * p.K * 2 + p.K * p.N * 2 + 2 * p.M * p.N * 2,
                          describe=plan.describe(p.M, p.N, p.K)))
        del p.A, p.B
    return items, "bf16"


def build_batched():
    """The batched example of the CUTLASS Python page: 16 independent fp16
    1024^3 GEMMs (A [16, M, K], B [16, K, N], D [16, M, N], RowMajor, beta 0)."""
    import torch
    import synthetic as syn
    import dense_gemm_epilogue_02_amd as g
    dev = torch.device("cuda:0")
    bs, M, N, K = 16, 1024, 1024, 1024
    probs = [syn.make_problem(M, N, K, dtype_ab="f16", dtype_cd="f16", seed=200 + b)
             for b in range(bs)]
    A = torch.stack([q.A for q in probs]).to(dev)
    B = torch.stack([q.B for q in probs]).to(dev)
    D = torch.empty((bs, M, N), dtype=torch.float16, device=dev)
    plan = g.Plan("f16", la="row", lb="row", lc="row")
    shape = type("S", (), dict(M=M, N=N, K=K))
    return [dict(name="batched16_f16_1024", p=shape, flops=2 * bs * M * N * K, plan=plan,
                 call=lambda: plan.run_batched(A, B, None, D, M, N, K, bs,
                                               (M * K, K * N, 0, M * N)),
                 bytes=2 * bs * (M * K + K * N + M * N),
                 describe=plan.describe_batched(M, N, K, bs))], "f16"


def build(workload):
    if workload == "layer_nn":
        return build_layer(["qkv", "o", "gate_up", "down"], lb="row")
    if workload == "batched16":
        return build_batched()
    if workload == "mx_layer":
        return build_mx_layer()
    if workload == "layer_residual":
        return build_layer_residual()
    if workload == "layer":
        return build_layer(["qkv", "o", "gate_up", "down"])
    if workload == "down":
        return build_layer(["down"])
    if workload == "fp16_1024_relu":
        return build_fp16_relu()
    if workload == "grouped64":
        return build_grouped()
    if workload == "fp8_decode":
        return build_fp8()
    if workload == "fp32_small":
        return build_fp32()
    raise SystemExit(f"unknown workload {workload}")


# ----------------------------------------------------------------- timing

def time_steps(items, steps, warmup):
    import torch
    for _ in range(warmup):
        for it in items:
            it["call"]()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()       # the launch stream of every call
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in items] for _ in range(steps)]
    t0 = time.perf_counter()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for s in range(steps):
        for i, it in enumerate(items):
            ev[s][i][0].record(stream)
            it["call"]()
            ev[s][i][1].record(stream)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = start.elapsed_time(end)
    per = [sum(ev[s][i][0].elapsed_time(ev[s][i][1]) for s in range(steps)) / steps
           for i in range(len(items))]
    return total_ms / steps, per, wall


def cpu_baseline(target_s: float = 15.0):
    """The oracle as it stands, on a row sample of the down-projection GEMM."""
    import numpy as np
    import oracle
    import synthetic as syn
    p = syn.config4("down", seed=3)
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    rows = max(1, threads)
    t0 = time.perf_counter()
    oracle.gemm(p, rows=list(range(rows)))
    dt = time.perf_counter() - t0
    # scale the sample to roughly target_s of CPU work
    scale = max(1, int(target_s / max(dt, 1e-3)))
    rows2 = min(p.M, rows * scale)
    t0 = time.perf_counter()
    oracle.gemm(p, rows=list(np.linspace(0, p.M - 1, rows2).astype(int)))
    dt2 = time.perf_counter() - t0
    flops = 2.0 * rows2 * p.N * p.K
    return {"value": flops / dt2 / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{rows2} of {p.M} rows of the down GEMM 4096x8192x28672 bf16 "
                      f"({flops / 1e9:.1f} GFLOP, {dt2:.1f} s wall, fp64 C loops, OpenMP)",
            "seconds": dt2}


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="layer", choices=WORKLOADS)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-tune", action="store_true",
                    help="skip the profiler step of the small / skinny workloads")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {args.gpus} is not supported "
              "(the GEMM path has no cross-GPU sharding).", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    items, dtype = build(args.workload)
    if not args.no_tune:
        # the library's profiler times every launch of each shape and caches
        # the fastest in the plan (untimed; the workloads without a tune step
        # keep the heuristics, which the profiler ranks first on them)
        for it in items:
            if "tune" in it:
                it["tune"]()
                it["describe"] = it["plan"].describe(it["p"].M, it["p"].N, it["p"].K)
                it["describe"]["tuned"] = True
    print(f"[bench] workload {args.workload}: {len(items)} launches per step; "
          f"{[it['describe'] for it in items]}", file=sys.stderr, flush=True)
    ms, per, wall = time_steps(items, args.steps, args.warmup)
    flops = sum(it["flops"] for it in items)
    tflops = flops / (ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[dtype]
    per_gemm = {}
    for it, d in zip(items, per):
        per_gemm[it["name"]] = {
            "us": round(d * 1e3, 2), "tflops": round(it["flops"] / (d * 1e-3) / 1e12, 1),
            "pct_peak": round(100 * it["flops"] / (d * 1e-3) / 1e12 / peak, 1),
            "hbm_gbs": round(it["bytes"] / (d * 1e-3) / 1e9, 1),
            "schedule": it["describe"].get("schedule"), "tile": it["describe"].get("tile"),
            "tuned": bool(it["describe"].get("tuned", False))}
    # dominant kernel: every launch of the default workload is the same kernel
    launch_flops = flops / len(items)
    launch_s = sum(per) / len(per) * 1e-3
    if args.workload == "fp8_decode":
        launch_bytes = sum(it["bytes"] for it in items) / len(items)
        roof = {"bound": "hbm", "achieved": round(launch_bytes / launch_s / 1e9, 1),
                "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": round(launch_flops / launch_s / 1e12, 1),
                "peak": peak, "unit": "TFLOP/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["traffic"] = load_traffic(args.workload)
    out = {
        "metric": METRIC, "value": round(tflops, 1), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dtype,
        "data": "synthetic (seeded; shapes and distributions of the workloads, no weights)",
        "config": {"workload": {"layer": "llama70b_like_layer_gemms_bf16_m4096",
                                "down": "down_proj_bf16_4096x8192x28672",
                                "fp16_1024_relu": "fp16_1024cubed_relu",
                                "grouped64": "grouped64_fp16_seed0",
                                "fp8_decode": "fp8_e4m3_decode_shapes",
                                "fp32_small": "fp32_128x64x256",
                                "mx_layer": "llama70b_like_layer_gemms_mxfp8_m4096",
                                "layer_residual": "o_and_down_proj_bf16_residual_add_m4096",
                                "batched16": "batched16_fp16_1024cubed",
                                "layer_nn": "llama70b_like_layer_gemms_bf16_m4096_rowmajor_b",
                                }[args.workload],
                   "gemms": {it["name"]: [it["p"].M, it["p"].N, it["p"].K] for it in items},
                   "layout": "A RowMajor, B ColumnMajor ([N,K]), D RowMajor"
                   if args.workload in ("layer", "down", "fp8_decode", "mx_layer",
                                        "layer_residual") else "all RowMajor"},
        "pct_peak": round(100 * tflops / peak, 2),
        "per_gemm": per_gemm,
        "roofline": roof,
        "timed_wall_s": round(wall, 3),
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline()
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
