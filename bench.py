#!/usr/bin/env python3
"""Benchmark of the gfx950 GEMM library on one MI355X.

Default workload (one "step"): the four bf16 GEMMs of a Llama-70B-like
transformer layer at M = 4096 tokens -- QKV 4096x10240x8192, O 4096x8192x8192,
gate/up 4096x57344x8192, down 4096x8192x28672 -- with A ~ N(0,1) RowMajor,
weights ~ N(0, 0.02^2) stored [N, K] (ColumnMajor B), fp32 accumulation, bf16 D.
The full-size inputs are drawn on the GPU (torch's generator; the parity tests
draw the same distributions on the host) and are resident in HBM before the
timed region starts.

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

# dense peaks at 2.4 GHz (256 CUs x 4 SIMDs): bf16/fp16 1024, fp8 2048, fp4
# 4096 FLOP per SIMD per cycle; fp32 through the MFMA pipe 157.3 TFLOP/s
PEAK_TFLOPS = {"bf16": 2516.6, "f16": 2516.6, "f8e4m3": 5033.2, "f4e2m1": 10066.3,
               "f32": 157.3}
DATASHEET_GHZ = 2.4
PEAK_HBM_GBS = 8000.0
METRIC = "GEMM TFLOP/s and % of MI355X MFMA peak per dtype, 1 GPU"

WORKLOADS = ("layer", "down", "fp16_1024_relu", "grouped64", "fp8_decode", "fp32_small",
             "mx_layer", "layer_residual", "batched16", "layer_nn", "mx4_layer",
             "fp32_ones_1024")

WORKLOAD_NAMES = {
    "layer": "llama70b_like_layer_gemms_bf16_m4096",
    "down": "down_proj_bf16_4096x8192x28672",
    "fp16_1024_relu": "fp16_1024cubed_relu",
    "grouped64": "grouped64_fp16_seed0",
    "fp8_decode": "fp8_e4m3_decode_shapes",
    "fp32_small": "fp32_128x64x256",
    "fp32_ones_1024": "fp32_all_ones_1024cubed",
    "mx_layer": "llama70b_like_layer_gemms_mxfp8_m4096",
    "mx4_layer": "llama70b_like_layer_gemms_mxfp4_m4096",
    "layer_residual": "o_and_down_proj_bf16_residual_add_m4096",
    "batched16": "batched16_fp16_1024cubed",
    "layer_nn": "llama70b_like_layer_gemms_bf16_m4096_rowmajor_b",
}


def source_hash() -> str:
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "dense_gemm_epilogue_02_amd", "csrc", "*"))):
        with open(f, "rb") as fh:
            h.update(os.path.basename(f).encode())
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_counters(workload: str):
    """The committed rocprofv3 counter summary of ``workload``
    (profiles/counters_<workload>.json, written by ``--summarize``), or None
    when it is missing or the kernel sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"counters_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        t = json.load(fh)
    if t.get("source_hash") != source_hash():
        return None
    return t


# ----------------------------------------------------------------- workloads

def build_layer(names, lb="col"):
    import torch
    import synthetic as syn
    import dense_gemm_epilogue_02_amd as g
    dev = torch.device("cuda:0")
    plan = g.Plan("bf16", la="row", lb=lb, lc="row")
    items = []
    for i, name in enumerate(names):
        M, N, K, A, B = syn.config4_device(name, dev, seed=i, lb=lb)
        D = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        shape = type("S", (), dict(M=M, N=N, K=K))
        items.append(dict(name=name, p=shape, flops=2 * M * N * K, plan=plan,
                          call=(lambda A=A, B=B, D=D, M=M, N=N, K=K:
                                plan.run(A, B, None, D, M, N, K, 1.0, 0.0)),
                          bytes=M * K * 2 + K * N * 2 + M * N * 2,
                          describe=plan.describe(M, N, K)))
    torch.cuda.synchronize()
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
    # the list is checked and packed once, as a serving loop would hold it
    prepared = plan.prepare_grouped(args, 0.0)
    return [dict(name="grouped64", p=probs[0], flops=flops, plan=plan,
                 call=lambda: plan.run_grouped(prepared, 1.0, 0.0), bytes=nbytes,
                 describe={"kernel": "grouped", "tile": "128x128", "problems": len(probs)})], "f16"


def build_fp8():
    """The six decode shapes; every shape has its own B (235 MB or 470 MB of
    e4m3), run back to back, so the 256 MB MALL never holds a B between its
    uses."""
    import torch
    import synthetic as syn
    import dense_gemm_epilogue_02_amd as g
    dev = torch.device("cuda:0")
    plan = g.Plan("f8e4m3", la="row", lb="col", lc="row")
    items = []
    for i, M in enumerate(syn.DECODE_MS):
        for j, (N, K) in enumerate(syn.DECODE_NK):
            A, B, s_a, s_b = syn.config5_device(M, N, K, dev, seed=10 * i + j)
            sa = torch.tensor([s_a], dtype=torch.float32, device=dev)
            sb = torch.tensor([s_b], dtype=torch.float32, device=dev)
            D = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            shape = type("S", (), dict(M=M, N=N, K=K))
            items.append(dict(name=f"fp8_{M}x{N}x{K}", p=shape, flops=2 * M * N * K, plan=plan,
                              call=(lambda A=A, B=B, D=D, sa=sa, sb=sb, M=M, N=N, K=K:
                                    plan.run(A, B, None, D, M, N, K, 1.0, 0.0, sa, sb)),
                              tune=(lambda A=A, B=B, D=D, M=M, N=N, K=K:
                                    plan.profile(A, B, None, D, M, N, K, 1.0, 0.0, iters=10)),
                              bytes=M * K + K * N + M * N * 2,
                              describe=plan.describe(M, N, K)))
    torch.cuda.synchronize()
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
    # a launch-bound problem run again and again on the same buffers: checked
    # and packed once (Plan.prepare), as a serving loop would hold it (the
    # plan's tuned choice still applies: it is looked up in every launch)
    call = plan.prepare(A, B, C, D, p.M, p.N, p.K, 1.0, 1.0)
    return [dict(name="fp32_128x64x256", p=p, flops=p.flops, plan=plan,
                 call=call,
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
        M, N, K, A, B = syn.config4_device(name, dev, seed=i)
        gen = torch.Generator(device=dev)
        gen.manual_seed(100 + i)
        X = torch.randn((M, N), generator=gen, device=dev).to(torch.bfloat16)
        D = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        shape = type("S", (), dict(M=M, N=N, K=K))
        items.append(dict(name=name + "_residual", p=shape, flops=2 * M * N * K, plan=plan,
                          call=(lambda A=A, B=B, D=D, X=X, M=M, N=N, K=K:
                                plan.run_aux(A, B, None, D, M, N, K, aux=X,
                                             aux_op="add", aux_pos="before")),
                          bytes=M * K * 2 + K * N * 2 + 2 * M * N * 2,
                          describe=plan.describe(M, N, K)))
    torch.cuda.synchronize()
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


def build_mx4_layer():
    """The four layer GEMMs in MXFP4 (e2m1 elements packed two per byte along
    K, E8M0 scales per 32 K elements)."""
    import torch
    import synthetic as syn
    import dense_gemm_epilogue_02_amd as g
    dev = torch.device("cuda:0")
    plan = g.Plan("f4e2m1", la="row", lb="col", lc="row")
    items = []
    for i, name in enumerate(("qkv", "o", "gate_up", "down")):
        M, N, K, A, B, xa, xb = syn.mx4_layer_device(name, dev, seed=i)
        D = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        shape = type("S", (), dict(M=M, N=N, K=K))
        items.append(dict(name=name, p=shape, flops=2 * M * N * K, plan=plan,
                          call=(lambda A=A, B=B, D=D, xa=xa, xb=xb, M=M, N=N, K=K:
                                plan.run_mx(A, B, None, D, M, N, K, xa, xb)),
                          bytes=(M * K + K * N) // 2 + M * N * 2 + (M + N) * (K // 32),
                          describe=plan.describe(M, N, K)))
    torch.cuda.synchronize()
    return items, "f4e2m1"


def build_fp32_ones():
    """The all-ones fp32 1024^3 GEMM with C = 1, alpha = beta = 1 (D = K + 1)."""
    import torch
    import synthetic as syn
    import dense_gemm_epilogue_02_amd as g
    dev = torch.device("cuda:0")
    p = syn.config1_ones()
    plan = g.Plan("f32", la="row", lb="row", lc="row")
    A, B, C = p.A.to(dev), p.B.to(dev), p.C.to(dev)
    D = torch.empty_like(C)
    return [dict(name="fp32_ones_1024", p=p, flops=p.flops, plan=plan,
                 call=lambda: plan.run(A, B, C, D, p.M, p.N, p.K, 1.0, 1.0),
                 tune=lambda: plan.profile(A, B, C, D, p.M, p.N, p.K, 1.0, 1.0, iters=20),
                 bytes=4 * 4 * 1024 * 1024,
                 describe=plan.describe(p.M, p.N, p.K))], "f32"


def build(workload):
    if workload == "mx4_layer":
        return build_mx4_layer()
    if workload == "fp32_ones_1024":
        return build_fp32_ones()
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


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def _oracle_rows_rate(p, threads: int, target_s: float):
    """Oracle FLOP/s on whole rows of ``p``: one pass of ``threads`` rows to
    size the sample, then about ``target_s`` seconds of rows spread over M."""
    import numpy as np
    import oracle
    rows = min(p.M, threads)
    t0 = time.perf_counter()
    oracle.gemm(p, rows=list(range(rows)))
    dt = time.perf_counter() - t0
    if dt >= target_s / 2 or rows == p.M:        # the sizing pass is sample enough
        return 2.0 * rows * p.N * p.K, dt, rows
    n = min(p.M, max(rows, int(rows * target_s / max(dt, 1e-4))))
    sel = np.unique(np.linspace(0, p.M - 1, n).astype(int))
    t0 = time.perf_counter()
    oracle.gemm(p, rows=list(sel))
    dt = time.perf_counter() - t0
    flops = 2.0 * sel.size * p.N * p.K
    return flops, dt, sel.size


def _per_config_rates(threads: int, target_s: float):
    """One bounded oracle sample per workload family; each keeps the
    workload's K, dtypes, layouts and value distribution, and bounds M (and,
    where the full operands would take long to draw on the host, N)."""
    import synthetic as syn
    out = {}

    def put(key, flops, dt, sample):
        out[key] = {"value": round(flops / dt / 1e9, 3), "unit": "GFLOP/s",
                    "seconds": round(dt, 2), "sample": sample}

    p = syn.config1()
    t0, reps = time.perf_counter(), 0
    while time.perf_counter() - t0 < target_s / 4 or reps == 0:
        import oracle
        oracle.gemm(p)
        reps += 1
    put("fp32_128x64x256", reps * p.flops, time.perf_counter() - t0,
        f"the whole 128x64x256 fp32 GEMM, {reps} times")
    p = syn.config1_ones()
    f, dt, n = _oracle_rows_rate(p, threads, target_s)
    put("fp32_ones_1024", f, dt, f"{n} of 1024 rows of the all-ones fp32 1024^3 GEMM")
    p = syn.config2()
    f, dt, n = _oracle_rows_rate(p, threads, target_s)
    put("fp16_1024_relu", f, dt, f"{n} of 1024 rows of the fp16 1024^3 ReLU GEMM")
    shapes = syn.config3_shapes()[:16]
    probs = syn.config3(shapes=shapes)
    import oracle
    t0, flops = time.perf_counter(), 0.0
    for q in probs:
        oracle.gemm(q, rows=list(range(min(q.M, 2))))
        flops += 2.0 * min(q.M, 2) * q.N * q.K
    put("grouped64", flops, time.perf_counter() - t0,
        "2 rows of each of the first 16 grouped fp16 problem shapes")
    p = syn.config5(16, 512, 28672)
    f, dt, n = _oracle_rows_rate(p, threads, target_s)
    put("fp8_decode", f, dt, f"{n} of 16 rows of an fp8 e4m3 16x512x28672 GEMM "
        "(the decode shape's K and distribution, 512 of its 8192 columns)")
    for key, elem in (("mx_layer", syn.F8), ("mx4_layer", syn.F4)):
        p = syn.make_mx_problem(8, 512, 28672, elem=elem, seed=3)
        f, dt, n = _oracle_rows_rate(p, threads, target_s)
        put(key, f, dt, f"{n} of 8 rows of an MX ({elem}) 8x512x28672 GEMM (the down "
            "projection's K, 512 of its 8192 columns)")
    return out


def cpu_baseline(workload: str, target_s: float = 10.0, per_config_s: float = 1.0):
    """The oracle as it stands: a row sample of the down-projection GEMM
    (the headline), plus one bounded sample per workload family."""
    import synthetic as syn
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    p = syn.config4("down", seed=3)
    flops, dt, n = _oracle_rows_rate(p, threads, target_s)
    del p
    per = _per_config_rates(threads, per_config_s)
    base = {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"{n} of 4096 rows of the down GEMM 4096x8192x28672 bf16 "
                      f"({flops / 1e9:.1f} GFLOP, {dt:.1f} s wall, fp64 C loops, OpenMP)",
            "seconds": round(dt, 2), "per_config": per}
    key = {"batched16": "fp16_1024_relu"}.get(workload, workload)
    if key in per:
        e = per[key]
        base.update(value=round(e["value"] / 1e3, 6), sample=e["sample"],
                    seconds=e["seconds"])
    return base


# ----------------------------------------------------------------- counters

KERNEL_TAG = {
    "layer": "gemm_bf16_tn", "down": "gemm_bf16_tn", "fp16_1024_relu": "gemm_f16_nn_relu",
    "grouped64": "gemm_grouped_f16_nn", "fp8_decode": "gemm_f8_tn", "fp32_small": "gemm_f32_nn",
    "fp32_ones_1024": "gemm_f32_nn", "mx_layer": "gemm_mxf8_tn", "mx4_layer": "gemm_mxf4_tn",
    "layer_residual": "gemm_bf16_tn_aux", "batched16": "gemm_f16_nn_batched",
    "layer_nn": "gemm_bf16_nn",
}
COPY_BYTES = 1 << 30     # the calibration copy of a recorded run


def record(path, args, items, dtype):
    """Write the launch table of this run (for --summarize) and run one plain
    1 GiB device copy after the timed region: FETCH_SIZE and WRITE_SIZE of
    that copy calibrate the counters in the same process."""
    import torch
    meta = {"workload": args.workload, "dtype": dtype, "steps": args.steps,
            "warmup": args.warmup, "argv": sys.argv[1:], "source_hash": source_hash(),
            "copy_bytes": COPY_BYTES,
            "items": [{"name": it["name"], "shape": [it["p"].M, it["p"].N, it["p"].K],
                       "flops": it["flops"], "bytes": it["bytes"],
                       "describe": it["describe"]} for it in items]}
    with open(path, "w") as fh:
        json.dump(meta, fh, indent=1)
    x = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda:0")
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    y.copy_(x)
    torch.cuda.synchronize()
    del x, y


def _is_gemm(name: str) -> bool:
    return "mg::" in name and "zero_u32" not in name


def _read_db(db):
    """(kernel rows ordered by start, per-dispatch counters) of one rocpd
    database: counters[dispatch_id] = {"name", "duration", counter: value}."""
    import sqlite3
    c = sqlite3.connect(db)
    rows = list(c.execute("select dispatch_id, name, duration, grid_x, workgroup_x, lds_size, "
                          "scratch_size, vgpr_count, accum_vgpr_count, sgpr_count "
                          "from kernels order by start"))
    cnt = {}
    try:
        for d, name, cn, v, dur in c.execute(
                "select dispatch_id, kernel_name, counter_name, value, duration "
                "from counters_collection order by dispatch_id"):
            e = cnt.setdefault(d, {"name": name, "duration": dur})
            e[cn] = e.get(cn, 0.0) + float(v)
    except sqlite3.OperationalError:
        pass
    c.close()
    return rows, cnt


def summarize(d: str, workload: str, outdir: str = None):
    """Turn the rocprofv3 databases of profile_bench.sh (kernel trace,
    FETCH_SIZE, WRITE_SIZE, clock + MFMA-busy passes over the same bench
    command) into profiles/counters_<workload>.json and a markdown summary."""
    import statistics as st
    meta = json.load(open(os.path.join(d, "items.json")))
    assert meta["workload"] == workload, (meta["workload"], workload)
    items = meta["items"]
    L = len(items)
    n_run = (meta["steps"] + meta["warmup"]) * L
    n_warm = meta["warmup"] * L
    cmds = open(os.path.join(d, "commands.txt")).read().strip() \
        if os.path.exists(os.path.join(d, "commands.txt")) else "(commands not recorded)"
    trace, pmc = None, {}
    for db in sorted(glob.glob(os.path.join(d, "*_results.db"))):
        rows, cnt = _read_db(db)
        if cnt:
            pmc[os.path.basename(db)[:-len("_results.db")]] = (rows, cnt)
        else:
            trace = rows
    out = {"workload": workload, "source_hash": meta["source_hash"], "dtype": meta["dtype"],
           "launches_per_step": L, "steps": meta["steps"], "warmup": meta["warmup"],
           "per_gemm": {it["name"]: {"shape": it["shape"], "flops": it["flops"],
                                     "algorithmic_bytes": it["bytes"]} for it in items}}
    md = [f"# {KERNEL_TAG[workload]} -- {WORKLOAD_NAMES[workload]}", "",
          "Commands (repo root, one MI355X; one rocprofv3 pass per counter group):", "", "```",
          cmds, "```", ""]
    peak = PEAK_TFLOPS[meta["dtype"]]
    if trace is not None:
        gemm = [r for r in trace if _is_gemm(r[1])][-n_run:]
        kinds = {}
        for r in trace:
            k = kinds.setdefault(r[1], [0, 0.0, r])
            k[0] += 1
            k[1] += r[2] / 1e3
        tot = sum(v[1] for v in kinds.values()) or 1.0
        md += ["Kernel trace (`--kernel-trace --stats`), every dispatch of the run:", "",
               "| kernel | calls | total us | avg us | % |", "|---|---|---|---|---|"]
        top = sorted(kinds.items(), key=lambda kv: -kv[1][1])
        for name, (cntk, t, r) in top[:12]:
            md.append(f"| `{name[:160]}` | {cntk} | {t:.1f} | {t / cntk:.1f} | {100 * t / tot:.2f} |")
        md += ["", "| GEMM kernel | grid (work-items) | wg | lds | vgpr | agpr | sgpr | scratch |",
               "|---|---|---|---|---|---|---|---|"]
        for name, (cntk, t, r) in top:
            if _is_gemm(name):
                md.append(f"| `{name[:160]}` | {r[3]} | {r[4]} | {r[5]} | {r[7]} | {r[8]} | "
                          f"{r[9]} | {r[6]} |")
        warm = gemm[n_warm:]
        for i, it in enumerate(items):
            ds = [r[2] / 1e3 for j, r in enumerate(warm) if j % L == i]
            out["per_gemm"][it["name"]]["trace_us"] = round(st.mean(ds), 2)
        mean_us = st.mean(r[2] / 1e3 for r in warm)
        mean_flops = st.mean(it["flops"] for it in items)
        mean_bytes = st.mean(it["bytes"] for it in items)
        out["launch"] = {"trace_us": round(mean_us, 2),
                         "tflops": round(mean_flops / (mean_us * 1e-6) / 1e12, 1),
                         "algorithmic_gbs": round(mean_bytes / (mean_us * 1e-6) / 1e9, 1)}
        md += ["", f"{len(gemm)} GEMM launches ({meta['warmup']} warm-up + {meta['steps']} timed "
               f"steps x {L}); the warm-up launches are excluded below.", "",
               "| GEMM | M x N x K | mean us | TFLOP/s | % of peak | algorithmic GB/s |",
               "|---|---|---|---|---|---|"]
        for it in items:
            us = out["per_gemm"][it["name"]]["trace_us"]
            tf = it["flops"] / (us * 1e-6) / 1e12
            md.append(f"| {it['name']} | {'x'.join(map(str, it['shape']))} | {us:.1f} | "
                      f"{tf:.1f} | {100 * tf / peak:.1f} | "
                      f"{it['bytes'] / (us * 1e-6) / 1e9:.0f} |")
        md += ["", f"Mean launch: {mean_us:.1f} us = {out['launch']['tflops']} TFLOP/s "
               f"({100 * out['launch']['tflops'] / peak:.1f} % of the {peak} TFLOP/s "
               f"{meta['dtype']} peak), {out['launch']['algorithmic_gbs']} GB/s of "
               "algorithmic bytes."]

    def gemm_dispatches(cnt):
        ids = [k for k in sorted(cnt) if _is_gemm(cnt[k]["name"])]
        return ids[-n_run:], ids[-1] if ids else None

    def copy_value(cnt, last, counter):
        vals = [e[counter] for k, e in sorted(cnt.items())
                if last is not None and k > last and "copy" in e["name"].lower() and counter in e]
        return max(vals) if vals else None

    fetch = pmc.get("fetch")
    write = pmc.get("write")
    cf = cw = None
    if fetch and write:
        (_, fc), (_, wc) = fetch, write
        fids, flast = gemm_dispatches(fc)
        wids, wlast = gemm_dispatches(wc)
        cf, cw = copy_value(fc, flast, "FETCH_SIZE"), copy_value(wc, wlast, "WRITE_SIZE")
        if not cf or not cw:
            md += ["", "(FETCH_SIZE / WRITE_SIZE runs lack the calibration copy: no traffic.)"]
    if fetch and write and cf and cw:
        copy_kib = meta["copy_bytes"] / 1024
        ff = copy_kib / cf if cf else None
        fw = copy_kib / cw if cw else None
        out["calibration"] = {"copy_bytes": meta["copy_bytes"], "copy_FETCH_SIZE_kib": cf,
                              "copy_WRITE_SIZE_kib": cw, "FETCH_SIZE": ff, "WRITE_SIZE": fw}
        md += ["", "HBM traffic (`--pmc FETCH_SIZE`, then `--pmc WRITE_SIZE`, in KiB per dispatch; "
               f"calibrated by the 1 GiB device copy the same run makes after its timed region: "
               f"FETCH_SIZE {cf:.0f} KiB, WRITE_SIZE {cw:.0f} KiB for {copy_kib:.0f} KiB "
               f"copied, so bytes = (FETCH_SIZE x {ff:.3f} + WRITE_SIZE x {fw:.3f}) x 1024). "
               "FETCH_SIZE counts L2 misses, some of which the MALL serves: an upper bound on "
               "HBM reads.", "",
               "| GEMM | FETCH_SIZE KiB | WRITE_SIZE KiB | calibrated bytes | algorithmic bytes | "
               "ratio |", "|---|---|---|---|---|---|"]
        tot = []
        for i, it in enumerate(items):
            f = st.mean(fc[k]["FETCH_SIZE"] for j, k in enumerate(fids) if j % L == i)
            w = st.mean(wc[k]["WRITE_SIZE"] for j, k in enumerate(wids) if j % L == i)
            hbm = (f * ff + w * fw) * 1024
            tot.append(hbm)
            e = out["per_gemm"][it["name"]]
            e.update(fetch_kib=round(f, 1), write_kib=round(w, 1), hbm_bytes=int(hbm),
                     traffic_ratio=round(hbm / it["bytes"], 3))
            md.append(f"| {it['name']} | {f:.0f} | {w:.0f} | {hbm / 1e9:.4f} GB | "
                      f"{it['bytes'] / 1e9:.4f} GB | {hbm / it['bytes']:.2f} |")
        out.setdefault("launch", {})["hbm_bytes"] = int(st.mean(tot))
        md += ["", f"Mean per launch: {st.mean(tot) / 1e9:.4f} GB (the bench line's "
               "`roofline.traffic`)."]
        if "trace_us" in out["launch"]:
            md.append(f"At the trace's mean launch time that is "
                      f"{st.mean(tot) / (out['launch']['trace_us'] * 1e-6) / 1e9:.0f} GB/s "
                      f"measured ({100 * st.mean(tot) / (out['launch']['trace_us'] * 1e-6) / 1e9 / PEAK_HBM_GBS:.1f} % "
                      f"of {PEAK_HBM_GBS:.0f} GB/s).")
    util = pmc.get("util")
    if util:
        _, uc = util
        uids, _ = gemm_dispatches(uc)
        md += ["", "Clock and matrix-core use (`--pmc GRBM_GUI_ACTIVE SQ_VALU_MFMA_BUSY_CYCLES "
               "SQ_BUSY_CYCLES`): GRBM_GUI_ACTIVE is summed over the 8 XCDs, so the "
               "achieved clock = value / 8 / dispatch duration; SQ_VALU_MFMA_BUSY_CYCLES is summed "
               "over the 1024 SIMDs, so MFMA busy = value / (per-XCD cycles x 1024). The "
               "clock-normalised fraction divides the achieved TFLOP/s by the peak scaled to "
               "the achieved clock.", "",
               "| GEMM | duration us | clock GHz | MFMA busy | TFLOP/s | at-clock fraction |",
               "|---|---|---|---|---|---|"]
        cyc_all, busy_all, dur_all, fl_all = 0.0, 0.0, 0.0, 0.0
        for i, it in enumerate(items):
            sel = [uc[k] for j, k in enumerate(uids) if j % L == i][meta["warmup"]:] or \
                  [uc[k] for j, k in enumerate(uids) if j % L == i]
            dur = st.mean(e["duration"] for e in sel) / 1e3        # us
            cyc = st.mean(e["GRBM_GUI_ACTIVE"] for e in sel) / 8
            busy = st.mean(e["SQ_VALU_MFMA_BUSY_CYCLES"] for e in sel)
            ghz = cyc / (dur * 1e3)
            tf = it["flops"] / (dur * 1e-6) / 1e12
            frac_clk = tf / (peak * ghz / DATASHEET_GHZ)
            e = out["per_gemm"][it["name"]]
            e.update(clock_ghz=round(ghz, 3), mfma_busy=round(busy / (cyc * 1024), 4),
                     frac_at_clock=round(frac_clk, 4), pmc_us=round(dur, 2))
            md.append(f"| {it['name']} | {dur:.1f} | {ghz:.3f} | {100 * busy / (cyc * 1024):.1f} % | "
                      f"{tf:.1f} | {frac_clk:.3f} |")
            cyc_all += cyc
            busy_all += busy
            dur_all += dur
            fl_all += it["flops"]
        ghz = cyc_all / (dur_all * 1e3)
        tf = fl_all / (dur_all * 1e-6) / 1e12
        out.setdefault("launch", {}).update(
            clock_ghz=round(ghz, 3), mfma_busy=round(busy_all / (cyc_all * 1024), 4),
            frac_at_clock=round(tf / (peak * ghz / DATASHEET_GHZ), 4))
        md += ["", f"All launches: {ghz:.3f} GHz, MFMA busy {100 * busy_all / (cyc_all * 1024):.1f} %, "
               f"{tf:.1f} TFLOP/s = {tf / peak:.3f} of the datasheet peak and "
               f"{tf / (peak * ghz / DATASHEET_GHZ):.3f} of the peak at the achieved clock."]
    md += ["", f"Kernel source hash (`bench.source_hash()`): `{meta['source_hash']}`."]
    if meta["source_hash"] != source_hash():
        md.append(f"(The sources have changed since: now `{source_hash()}`.)")
    tag = KERNEL_TAG[workload]
    outdir = outdir or os.path.join(ROOT, "profiles")
    os.makedirs(outdir, exist_ok=True)
    with open(os.path.join(outdir, f"counters_{workload}.json"), "w") as fh:
        json.dump(out, fh, indent=1)
    with open(os.path.join(outdir, f"{tag}__{workload}.md"), "w") as fh:
        fh.write("\n".join(md) + "\n")
    print(json.dumps(out.get("launch", {})))


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="layer", choices=WORKLOADS)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-tune", action="store_true",
                    help="skip the profiler step of the small / skinny workloads")
    ap.add_argument("--record", metavar="JSON",
                    help="write the launch table here and run a 1 GiB calibration copy "
                         "after the timed region (for counter runs)")
    ap.add_argument("--summarize", metavar="DIR",
                    help="no GPU: turn the rocprofv3 databases in DIR into profiles/ summaries")
    ap.add_argument("--profiles-dir", metavar="DIR", default=None,
                    help="where --summarize writes (default: profiles/)")
    args = ap.parse_args()
    if args.summarize:
        summarize(args.summarize, args.workload, args.profiles_dir)
        return
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
    if args.record:
        record(args.record, args, items, dtype)
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
    cnt = load_counters(args.workload)
    launch = (cnt or {}).get("launch", {})
    roof["traffic"] = launch.get("hbm_bytes")
    if "clock_ghz" in launch and roof["bound"] == "mfma":
        # achieved clock and MFMA busy from the committed counter run of the same
        # kernels; the fraction of the peak at that clock uses this run's time
        roof["sclk_ghz"] = launch["clock_ghz"]
        roof["mfma_busy"] = launch["mfma_busy"]
        roof["frac_at_sclk"] = round(roof["achieved"] / (peak * launch["clock_ghz"]
                                                          / DATASHEET_GHZ), 4)
    if roof["traffic"] is not None and roof["bound"] == "hbm":
        roof["traffic_gbs"] = round(roof["traffic"] / launch_s / 1e9, 1)
    out = {
        "metric": METRIC, "value": round(tflops, 1), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dtype,
        "data": "synthetic (seeded; shapes and distributions of the workloads, no weights)",
        "config": {"workload": WORKLOAD_NAMES[args.workload],
                   "gemms": {it["name"]: [it["p"].M, it["p"].N, it["p"].K] for it in items},
                   "layout": "A RowMajor, B ColumnMajor ([N,K]), D RowMajor"
                   if args.workload in ("layer", "down", "fp8_decode", "mx_layer", "mx4_layer",
                                        "layer_residual") else "all RowMajor"},
        "pct_peak": round(100 * tflops / peak, 2),
        "per_gemm": per_gemm,
        "roofline": roof,
        "timed_wall_s": round(wall, 3),
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(args.workload)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
