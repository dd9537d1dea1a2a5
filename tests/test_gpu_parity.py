"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bars: bit-exact on integer-valued data; otherwise the tolerances of
oracle.acceptance (fp32: 1e-5 S + 1e-6; fp16/bf16: 2 ulp + 2e-3 S; fp8 inputs:
2 ulp + 1.5e-2 S). Full-size workloads are checked on sampled outputs that the
oracle computes one by one, in the launch configuration the benchmark uses.
"""
import itertools
import os

import numpy as np
import pytest
import torch

import dense_gemm_epilogue_02_amd as g
import oracle
from oracle import acceptance
import synthetic as syn
from gpu_util import (DEV, check_guards, device_operands, full_size_samples, logical, make_out,
                      run, scales)

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
LAYOUTS = list(itertools.product(("row", "col"), repeat=3))
S, T = g.Schedule, g.Tile


def close(got, p, relu=False, what="", act=None):
    r = oracle.gemm(p, relu=relu, act=act)
    return acceptance.check_close(got, r.ref, r.S, p.dtype_ab, p.dtype_cd, what)


def exact(got, p, relu=False, what="", act=None):
    r = oracle.gemm(p, relu=relu, act=act)
    acceptance.check_exact(got, r.d_exact, what)


# ------------------------------------------------------------ worked examples

def _golden(name):
    kv = {}
    for line in open(os.path.join(GOLDEN, name)):
        line = line.strip()
        if line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    return kv


@pytest.mark.parametrize("name", ["ones_fp16_128.txt", "ones_fp16_1024.txt"])
def test_golden_ones(name):
    kv = _golden(name)
    M, N, K = int(kv["M"]), int(kv["N"]), int(kv["K"])
    p = syn.make_problem(M, N, K, dtype_ab=kv["dtype"], dtype_cd=kv["dtype"], dist_a="ones",
                         dist_b="ones", dist_c="ones", alpha=float(kv["alpha"]),
                         beta=float(kv["beta"]))
    got = run(p)
    assert (got == float(kv["expect_all"])).all()


# ------------------------------------------------------------ the workloads

@pytest.mark.parametrize("sched", [S.AUTO, S.DATA_PARALLEL, S.STREAM_K])
def test_config1_fp32_small(sched):
    p = syn.config1()
    close(run(p, schedule=sched), p, what=f"fp32 128x64x256 {sched.name}")


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_config1_ones_closed_form(dtype):
    p = syn.config1_ones(1024, dtype)
    got = run(p)
    want = oracle.decode(dtype, oracle.encode(dtype, [1025.0]))[0]   # bf16: 1024
    assert (got == want).all()


def test_config2_fp16_relu_full():
    p = syn.config2()
    got = run(p, relu=True)
    assert (got >= 0).all()
    close(got, p, relu=True, what="fp16 1024^3 relu")


@pytest.mark.parametrize("sched", [S.AUTO, S.DATA_PARALLEL, S.STREAM_K])
def test_config2_schedules(sched):
    p = syn.config2(n=512)
    close(run(p, relu=True, schedule=sched), p, relu=True, what=f"fp16 512^3 {sched.name}")


def describe_of(p, relu=False):
    """What a run of p would launch (host-only; the heuristics' choice)."""
    plan = g.Plan(p.dtype_ab, p.dtype_cd, p.la, p.lb, p.lc, relu)
    try:
        return plan.describe(p.M, p.N, p.K)
    finally:
        plan.close()


def check_full_size(got, p, seed, what):
    """Every output written (D starts as NaN), and one oracle entry in every
    32 x 32 block plus the corners of every tile compared."""
    assert np.isfinite(got).all(), f"{what}: unwritten (NaN) outputs"
    ii, jj = full_size_samples(p.M, p.N, seed, describe_of(p))
    r = oracle.gemm_entries(p, ii, jj)
    acceptance.check_close(got[ii, jj], r.ref, r.S, p.dtype_ab, p.dtype_cd, what)
    return len(ii)


@pytest.mark.parametrize("name", ["qkv", "o", "down", "gate_up"])
def test_config4_layer_gemm_every_block(name):
    p = syn.config4(name)
    got = run(p)
    n = check_full_size(got, p, 1, f"layer {name}")
    assert n >= (p.M // 32) * (p.N // 32)


def test_config4_row_major_b_every_block():
    p = syn.config4("o", lb="row")
    got = run(p)
    check_full_size(got, p, 2, "layer o, RowMajor B")


@pytest.mark.parametrize("M", syn.DECODE_MS)
@pytest.mark.parametrize("NK", syn.DECODE_NK)
def test_config5_fp8_every_block(M, NK):
    N, K = NK
    p = syn.config5(M, N, K)
    got = run(p)
    check_full_size(got, p, 3, f"fp8 {M}x{N}x{K}")


def test_config5_fp8_small_full():
    p = syn.config5(64, 1024, 2048, seed=4)
    close(run(p), p, what="fp8 64x1024x2048")


# ------------------------------------------------------------ bit-exact sweeps

FAMS = [("f32", "f32"), ("f16", "f16"), ("bf16", "bf16"), ("f8e4m3", "bf16")]
TILES = [T.T256x256, T.T128x128, T.T64x256, T.T32x256, T.GENERIC, T.WHOLEK]


def _int_problem(dab, dcd, la, lb, lc, M=304, N=272, K=208, seed=0, beta=1.0):
    # |sum| must stay exact in the output type: bf16 holds integers to 256
    lo, hi = (-1, 1) if dcd == "bf16" else (-2, 2)
    return syn.integer_problem(M, N, K, dtype_ab=dab, dtype_cd=dcd, la=la, lb=lb, lc=lc,
                               lo=lo, hi=hi, beta=beta, seed=seed)


@pytest.mark.parametrize("dab,dcd", FAMS)
@pytest.mark.parametrize("la,lb,lc", LAYOUTS)
@pytest.mark.parametrize("tile", TILES)
def test_integer_exact_all_layouts_tiles(dab, dcd, la, lb, lc, tile):
    p = _int_problem(dab, dcd, la, lb, lc)
    exact(run(p, tile=tile, schedule=S.DATA_PARALLEL), p,
          what=f"{dab} {la}{lb}{lc} {tile.name}")


@pytest.mark.parametrize("dab,dcd", FAMS)
@pytest.mark.parametrize("sched", [S.STREAM_K, S.HYBRID])
@pytest.mark.parametrize("tile", [T.T256x256, T.T128x128, T.T32x256])
@pytest.mark.parametrize("relu", [False, True])
def test_integer_exact_stream_k(dab, dcd, sched, tile, relu):
    p = _int_problem(dab, dcd, "row", "col", "row", M=544, N=528, K=1024, seed=5)
    got = run(p, relu=relu, tile=tile, schedule=sched, sk_grid=37 if sched == S.STREAM_K else 16)
    exact(got, p, relu=relu, what=f"{dab} {sched.name} {tile.name}")


@pytest.mark.parametrize("dab,dcd", FAMS)
@pytest.mark.parametrize("tile", [T.T128x128, T.T64x256, T.T32x256])
@pytest.mark.parametrize("relu", [False, True])
@pytest.mark.parametrize("lb", ["col", "row"])
def test_integer_exact_split_k(dab, dcd, tile, relu, lb):
    # few tiles, long ragged K: units of 8+ k-tiles, the first ones one longer
    p = _int_problem(dab, dcd, "row", lb, "row", M=200, N=272, K=2064, seed=11)
    got = run(p, relu=relu, tile=tile, schedule=S.SPLIT_K)
    exact(got, p, relu=relu, what=f"{dab} split-K {tile.name} lb={lb}")


@pytest.mark.parametrize("dab,dcd", FAMS)
@pytest.mark.parametrize("la,lb,lc", [("row", "row", "row"), ("col", "col", "col"),
                                      ("row", "col", "row"), ("col", "row", "col")])
def test_random_tolerance(dab, dcd, la, lb, lc):
    p = syn.make_problem(336, 400, 520, dtype_ab=dab, dtype_cd=dcd, la=la, lb=lb, lc=lc,
                         dist_c="normal", alpha=0.75, beta=-0.5, seed=7)
    for sched in (S.DATA_PARALLEL, S.STREAM_K, S.SPLIT_K):
        close(run(p, relu=True, schedule=sched), p, relu=True,
              what=f"{dab} {la}{lb}{lc} {sched.name}")


# ------------------------------------------------------------ stream-K

@pytest.mark.parametrize("M,N,K,tile,sched,sk_grid", [
    # AUTO resolves to hybrid with fewer stream-K iterations than workgroups
    (4352, 4096, 256, T.AUTO, S.AUTO, 0),        # 1088 tiles of 128^2 (K < 2048): 64 stream-K, ipt 4
    (3072, 3200, 256, T.T128x128, S.HYBRID, 0),  # 600 tiles of 128^2 over 2/CU
    (4352, 4096, 512, T.T256x256, S.HYBRID, 0),  # ipt 8: 128 iterations
    (2304, 2560, 256, T.T256x256, S.HYBRID, 0),  # 90 tiles < grid: resolves to stream-K
    (1024, 1280, 384, T.T128x128, S.STREAM_K, 200),
    (4352, 4352, 256, T.T256x256, S.HYBRID, 100),   # explicit grid, remainder of 89 tiles
])
def test_integer_exact_hybrid_few_iterations(M, N, K, tile, sched, sk_grid):
    """Stream-K remainders whose iterations number fewer than the grid
    (every workgroup must still own a non-empty range): NaN-prefilled D,
    compared with the oracle in full, bit-exact."""
    p = _int_problem("bf16", "bf16", "row", "col", "row", M=M, N=N, K=K, seed=M + K)
    plan = g.Plan("bf16", la="row", lb="col", lc="row")
    plan.set_config(sched, tile, sk_grid)
    d = plan.describe(M, N, K)
    if sched == S.AUTO:
        assert d["schedule"] == "hybrid" and d["sk_iters"] < d["grid"], d
    assert d["sk_grid"] <= max(d["sk_iters"], 1), d
    got = run(p, plan=plan, schedule=sched, tile=tile, sk_grid=sk_grid)
    # twice on one plan: the arrival counters must be left clean
    got2 = run(p, plan=plan, schedule=sched, tile=tile, sk_grid=sk_grid)
    plan.close()
    assert np.isfinite(got).all()
    exact(got, p, what=f"hybrid {M}x{N}x{K} {d}")
    assert np.array_equal(got, got2)


def test_stream_k_deterministic_and_equivalent():
    p = syn.make_problem(512, 512, 4096, dtype_ab="bf16", dtype_cd="bf16", lb="col", seed=8)
    dp = run(p, schedule=S.DATA_PARALLEL, tile=T.T128x128)
    for grid in (7, 64, 256):
        a = run(p, schedule=S.STREAM_K, tile=T.T128x128, sk_grid=grid)
        b = run(p, schedule=S.STREAM_K, tile=T.T128x128, sk_grid=grid)
        assert np.array_equal(a, b), f"stream-K grid {grid} not bitwise repeatable"
        close(a, p, what=f"stream-K grid {grid}")
    close(dp, p, what="data-parallel")


@pytest.mark.parametrize("grid", [0, 12, 24])
def test_split_k_deterministic_and_close(grid):
    # fp8 decode-like: 16 rows, 4 column tiles, K = 8192 (64 k-tiles of 128)
    p = syn.make_problem(16, 1024, 8192, dtype_ab="f8e4m3", dtype_cd="bf16", lb="col",
                         dist_c="normal", beta=0.5, seed=12)
    a = run(p, schedule=S.SPLIT_K, tile=T.T64x256, sk_grid=grid)
    b = run(p, schedule=S.SPLIT_K, tile=T.T64x256, sk_grid=grid)
    assert np.array_equal(a, b), f"split-K grid {grid} not bitwise repeatable"
    close(a, p, what=f"split-K grid {grid}")


def test_stream_k_matches_dp_on_integers():
    p = _int_problem("bf16", "bf16", "row", "col", "row", M=256, N=256, K=2048, seed=9)
    dp = run(p, schedule=S.DATA_PARALLEL, tile=T.T128x128)
    sk = run(p, schedule=S.STREAM_K, tile=T.T128x128, sk_grid=100)
    assert np.array_equal(dp, sk)
    exact(sk, p)


def test_plan_reuse_across_shapes_and_workspace_growth():
    plan = g.Plan("bf16", la="row", lb="col", lc="row")
    for (M, N, K) in ((64, 64, 256), (512, 512, 2048), (1000, 776, 1032), (128, 256, 64)):
        p = syn.make_problem(M, N, K, dtype_ab="bf16", dtype_cd="bf16", lb="col", seed=M)
        close(run(p, plan=plan, schedule=S.STREAM_K), p, what=f"reuse {M}x{N}x{K}")
    plan.close()


# ------------------------------------------------------------ grouped

def _grouped_run(plan, probs, alpha=1.0, beta=0.0):
    ops, outs, problems = [], [], []
    for p in probs:
        A, B, C = device_operands(p)
        buf, D = make_out(p)
        ops.append((A, B, C, buf))
        outs.append(D)
        problems.append((p.M, p.N, p.K, A, B, C, D))
    print(f"[gpu] grouped {len(probs)} problems", flush=True)
    plan.run_grouped(problems, alpha, beta)
    torch.cuda.synchronize()
    return [logical(D, p) for D, p in zip(outs, probs)]


def test_grouped_small_full_oracle():
    shapes = [(32, 128, 128), (96, 256, 512), (160, 512, 256), (544, 128, 1024),
              (64, 1024, 128), (2048, 256, 256), (0, 128, 128), (224, 128, 0)]
    probs = syn.config3(seed=11, shapes=shapes)
    plan = g.Plan("f16", la="row", lb="row", lc="row")
    outs = _grouped_run(plan, probs)
    for p, got in zip(probs, outs):
        close(got, p, what=f"grouped {p.M}x{p.N}x{p.K}")
    plan.close()


def test_grouped_config3_every_block():
    """The 64-problem grouped launch the benchmark times: every D fully
    written, one oracle entry per 32 x 32 block of every problem, and rows 0,
    M/2 and M-1 of every problem in full."""
    probs = syn.config3()
    plan = g.Plan("f16", la="row", lb="row", lc="row")
    outs = _grouped_run(plan, probs)
    for q, (p, got) in enumerate(zip(probs, outs)):
        what = f"grouped #{q} {p.M}x{p.N}x{p.K}"
        assert np.isfinite(got).all(), f"{what}: unwritten (NaN) outputs"
        ii, jj = full_size_samples(p.M, p.N, 100 + q)
        r = oracle.gemm_entries(p, ii, jj)
        acceptance.check_close(got[ii, jj], r.ref, r.S, "f16", "f16", what)
        rows = [0, p.M // 2, p.M - 1]
        r = oracle.gemm(p, rows=rows)
        acceptance.check_close(got[rows], r.ref, r.S, "f16", "f16", what + " rows")
    plan.close()


def test_grouped_equals_loop_of_singles_bitwise():
    probs = syn.config3(seed=12, count=10)
    plan = g.Plan("f16", la="row", lb="row", lc="row", relu=True)
    outs = _grouped_run(plan, probs)
    for p, got in zip(probs, outs):
        single = run(p, relu=True, schedule=S.DATA_PARALLEL, tile=T.T128x128)
        assert np.array_equal(got, single), f"grouped != single for {p.M}x{p.N}x{p.K}"
    plan.close()


def test_grouped_integer_exact_mixed_alignment():
    shapes = [(128, 128, 64), (40, 72, 24), (256, 136, 96), (33, 17, 9)]
    probs = [_int_problem("bf16", "bf16", "row", "row", "row", M=m, N=n, K=k, seed=i)
             for i, (m, n, k) in enumerate(shapes)]
    plan = g.Plan("bf16", la="row", lb="row", lc="row")
    outs = _grouped_run(plan, probs, beta=1.0)
    for p, got in zip(probs, outs):
        exact(got, p, what=f"grouped int {p.M}x{p.N}x{p.K}")
    plan.close()


def test_grouped_repeated_and_changed_problem_lists():
    """Back-to-back grouped calls with the same list reuse the uploaded
    descriptors; a changed list (another output, another shape) must not:
    every call's outputs are compared with the oracle, NaN-prefilled."""
    probs = syn.config3(seed=21, count=6)
    plan = g.Plan("f16", la="row", lb="row", lc="row")
    ops = [device_operands(p) for p in probs]
    outs = [make_out(p) for p in probs]

    def call(order):
        for i in order:
            outs[i][1].fill_(float("nan"))
        plan.run_grouped([(probs[i].M, probs[i].N, probs[i].K, ops[i][0], ops[i][1], None,
                           outs[i][1]) for i in order], 1.0, 0.0)
        torch.cuda.synchronize()
        for i in order:
            close(logical(outs[i][1], probs[i]), probs[i], what=f"grouped repeat #{i}")
            check_guards(outs[i][0], probs[i])

    call(range(6))
    call(range(6))           # same list: descriptors reused
    call(range(6))
    call([0, 2, 4])          # a different list
    out5 = make_out(probs[5])
    outs[5] = out5           # same shapes, another output tensor
    call(range(6))
    call(range(6))
    plan.close()


@pytest.mark.parametrize("dab", ["bf16", "f16"])
@pytest.mark.parametrize("la,lb", [("row", "col"), ("row", "row"), ("col", "col"), ("col", "row")])
def test_grouped_two_tile_classes_integer_exact(dab, la, lb):
    """Problems that take 256x256 tiles (little padding) and 128x128 tiles
    (M or N far from a multiple of 256) in one grouped call, two launches;
    ragged M, N and K tails; every operand layout."""
    shapes = [(768, 512, 136),    # 256x256 class, K tail
              (520, 264, 64),     # 128x128 class
              (256, 1024, 72),    # 256x256 class
              (96, 128, 40),      # 128x128 class
              (512, 1000, 200),   # 256x256 class, ragged N
              (512, 776, 200)]    # 128x128 class (256x256 would pad over 1/8 more)
    probs = [_int_problem(dab, dab, la, lb, "row", M=m, N=n, K=k, seed=40 + i)
             for i, (m, n, k) in enumerate(shapes)]
    plan = g.Plan(dab, la=la, lb=lb, lc="row")
    outs = _grouped_run(plan, probs, beta=1.0)
    for p, got in zip(probs, outs):
        exact(got, p, what=f"grouped {dab} {la}/{lb} {p.M}x{p.N}x{p.K}")
    plan.close()


def test_grouped_prepared_list_matches_and_guards():
    """A problem list checked and packed once (Plan.prepare_grouped) runs
    bitwise like the plain list, repeatedly; it refuses another plan and a
    beta that would read an unchecked C."""
    probs = [_int_problem("f16", "f16", "row", "row", "row", M=m, N=n, K=k, seed=60 + i)
             for i, (m, n, k) in enumerate([(300, 200, 64), (64, 520, 136), (1, 33, 8), (257, 256, 512)])]
    plan = g.Plan("f16", la="row", lb="row", lc="row")
    ops = [device_operands(p) for p in probs]
    a_out = [make_out(p) for p in probs]
    b_out = [make_out(p) for p in probs]
    plan.run_grouped([(p.M, p.N, p.K, o[0], o[1], o[2], d[1]) for p, o, d in zip(probs, ops, a_out)],
                     1.0, 1.0)
    prep = plan.prepare_grouped([(p.M, p.N, p.K, o[0], o[1], o[2], d[1])
                                 for p, o, d in zip(probs, ops, b_out)], 1.0)
    for _ in range(3):
        plan.run_grouped(prep, 1.0, 1.0)
    torch.cuda.synchronize()
    for p, (ba, Da), (bb, Db) in zip(probs, a_out, b_out):
        assert torch.equal(Da, Db)
        exact(logical(Db, p), p, what=f"prepared grouped {p.M}x{p.N}x{p.K}")
        check_guards(bb, p)
    prep0 = plan.prepare_grouped([(p.M, p.N, p.K, o[0], o[1], None, d[1])
                                  for p, o, d in zip(probs, ops, b_out)], 0.0)
    with pytest.raises(ValueError):
        plan.run_grouped(prep0, 1.0, 1.0)
    other = g.Plan("f16", la="row", lb="row", lc="row")
    with pytest.raises(ValueError):
        other.run_grouped(prep, 1.0, 1.0)
    other.close()
    plan.close()


def test_grouped_many_problems_tile_queue_integer_exact():
    """150 problems of uneven cost (K from 8 to 1032, M and N from 1 to 300):
    more tiles than the persistent grid, so most tiles come from the per-XCD
    claim queues; three calls in a row (the queue words reset themselves at
    the end of each launch) and a plain single GEMM in between on the same
    plan. Every output exact, NaN-prefilled, guards intact."""
    rng = np.random.default_rng(77)
    shapes = [(int(rng.integers(1, 301)), int(rng.integers(1, 301)), int(rng.integers(1, 130)) * 8)
              for _ in range(150)]
    probs = [_int_problem("f16", "f16", "row", "row", "row", M=m, N=n, K=k, seed=500 + i)
             for i, (m, n, k) in enumerate(shapes)]
    want = [oracle.gemm(p).d_exact for p in probs]
    plan = g.Plan("f16", la="row", lb="row", lc="row")
    ops = [device_operands(p) for p in probs]
    outs = [make_out(p) for p in probs]
    for rep in range(3):
        for buf, D in outs:
            D.fill_(float("nan"))
        print(f"[gpu] grouped 150 problems, call {rep}", flush=True)
        plan.run_grouped([(p.M, p.N, p.K, o[0], o[1], o[2], d[1])
                          for p, o, d in zip(probs, ops, outs)], 1.0, 1.0)
        torch.cuda.synchronize()
        for p, w, (buf, D) in zip(probs, want, outs):
            acceptance.check_exact(logical(D, p), w, f"grouped queue call {rep} {p.M}x{p.N}x{p.K}")
            check_guards(buf, p)
        if rep == 1:   # a single GEMM on the same plan between grouped calls
            q = _int_problem("f16", "f16", "row", "row", "row", M=300, N=200, K=64, seed=9)
            exact(run(q, plan=plan), q, what="single between grouped calls")
    plan.close()


# ------------------------------------------------------------ edge cases

def test_k_zero_gives_beta_c():
    p = syn.make_problem(100, 60, 0, dtype_ab="bf16", dtype_cd="bf16", dist_c="normal",
                         beta=2.0, seed=13)
    exact(run(p, relu=True), p, relu=True)


def test_empty_outputs_are_no_ops():
    for (M, N) in ((0, 16), (16, 0)):
        plan = g.Plan("f16")
        plan.run(None, None, None, None, M, N, 8)
        plan.close()


def test_in_place_d_equals_c():
    p = syn.make_problem(200, 152, 96, dtype_ab="f16", dtype_cd="f16", dist_c="normal",
                         beta=1.0, seed=14)
    close(run(p, in_place=True), p, what="in place")


def test_beta_zero_ignores_nan_c():
    p = syn.make_problem(128, 128, 64, dtype_ab="bf16", dtype_cd="bf16", dist_c="normal",
                         beta=0.0, seed=15)
    p.C = torch.full_like(p.C, float("nan"))
    got = run(p)
    assert np.isfinite(got).all()
    close(got, p)


def test_misaligned_operand_uses_generic_and_matches():
    p = syn.make_problem(96, 80, 64, dtype_ab="bf16", dtype_cd="bf16", dist_c="normal",
                         beta=1.0, seed=16)
    A, B, C = device_operands(p)
    A2 = torch.empty(p.M * p.K + 1, dtype=A.dtype, device=DEV)
    A2[1:] = A.reshape(-1)
    Ash = A2[1:]                         # 2-byte aligned base
    plan = g.Plan("bf16")
    # aligned operands get a vector-load kernel (the whole-K one at this size);
    # the 2-byte aligned A leaves the scalar-load kernel
    assert plan.describe(p.M, p.N, p.K)["kernel"] in ("tile", "wholek")
    got = run(p, plan=plan, operands=(Ash, B, C))
    close(got, p, what="misaligned A")
    plan.close()


@pytest.mark.parametrize("dab,dcd", FAMS)
def test_odd_sizes_generic(dab, dcd):
    p = _int_problem(dab, dcd, "row", "row", "row", M=37, N=29, K=13, seed=17)
    exact(run(p), p)


def test_alpha_two_doubles_bitwise_and_relu_fusion():
    p = syn.make_problem(256, 256, 512, dtype_ab="bf16", dtype_cd="bf16", dist_c="normal",
                         beta=1.0, seed=18)
    lin = run(p, schedule=S.DATA_PARALLEL, tile=T.T128x128)
    fused = run(p, relu=True, schedule=S.DATA_PARALLEL, tile=T.T128x128)
    assert np.array_equal(fused, np.maximum(lin, 0.0))
    p.alpha, p.beta = 2.0, 2.0
    dbl = run(p, schedule=S.DATA_PARALLEL, tile=T.T128x128)
    assert np.array_equal(dbl, 2.0 * lin)


def test_large_k_beyond_32bit_tile_span_uses_generic():
    K = (1 << 25) + 64
    p = syn.make_problem(2, 8, K, dtype_ab="bf16", dtype_cd="bf16", lb="col", seed=19)
    plan = g.Plan("bf16", lb="col")
    d = plan.describe(p.M, p.N, p.K)
    assert d["kernel"] == "generic" and "32-bit" in d["generic_reason"]
    close(run(p, plan=plan), p, what="K = 2^25 + 64")
    plan.close()


def test_fp8_scales_read_on_device():
    p = syn.integer_problem(64, 256, 256, dtype_ab="f8e4m3", dtype_cd="bf16", with_c=False,
                            lo=-1, hi=1, seed=20)
    p.scale_a, p.scale_b = 0.5, 0.25
    exact(run(p), p)


# ------------------------------------------------------------ bias + activations

@pytest.mark.parametrize("dab,dcd", FAMS)
@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("act", ["linear", "relu"])
def test_bias_integer_exact(dab, dcd, tile, act):
    # RowMajor C/D (vector epilogue on interior tiles), ragged edges
    p = _int_problem(dab, dcd, "row", "col", "row", M=272, N=304, K=192, seed=31)
    p.bias = syn.cast(np.random.default_rng(32).integers(-2, 3, p.N).astype(np.float32), dcd)
    got = run(p, tile=tile, schedule=S.DATA_PARALLEL, act=act)
    exact(got, p, act="identity" if act == "linear" else act, what=f"{dab} {tile.name} {act}")


@pytest.mark.parametrize("dab,dcd", FAMS)
@pytest.mark.parametrize("sched", [S.STREAM_K, S.SPLIT_K])
def test_bias_integer_exact_split_schedules_col_c(dab, dcd, sched):
    # the epilogue after a partial-tile fixup, ColumnMajor C/D (element path)
    p = _int_problem(dab, dcd, "row", "col", "col", M=200, N=264, K=1024, seed=33)
    p.bias = syn.cast(np.random.default_rng(34).integers(-2, 3, p.N).astype(np.float32), dcd)
    got = run(p, tile=T.T128x128, schedule=sched, act="relu", relu=True)
    exact(got, p, relu=True, what=f"{dab} {sched.name} col C")


@pytest.mark.parametrize("dab,dcd", FAMS)
@pytest.mark.parametrize("act", ["sigmoid", "tanh"])
@pytest.mark.parametrize("lb", ["col", "row"])
def test_sigmoid_tanh_with_bias(dab, dcd, act, lb):
    p = syn.make_problem(336, 400, 520, dtype_ab=dab, dtype_cd=dcd, lb=lb, dist_c="normal",
                         alpha=0.05, beta=0.5, dist_bias="normal", seed=35)
    for tile in (T.AUTO, T.T32x256, T.GENERIC):
        close(run(p, act=act, tile=tile), p, act=act, what=f"{dab} {act} lb={lb} {tile.name}")


def test_misaligned_bias_uses_element_epilogue():
    p = syn.make_problem(256, 512, 256, dtype_ab="bf16", dtype_cd="bf16", lb="col",
                         dist_bias="normal", seed=36)
    a = run(p, act="relu", relu=True, tile=T.T256x256, schedule=S.DATA_PARALLEL)
    b = run(p, act="relu", relu=True, tile=T.T256x256, schedule=S.DATA_PARALLEL, bias_offset=1)
    assert np.array_equal(a, b)     # same arithmetic, element-wise stores
    close(b, p, relu=True, what="misaligned bias")


def test_bias_without_activation_equals_shifted_linear():
    # D(bias) - D(no bias) == bias[n] exactly on integer data, every row
    p = _int_problem("f16", "f16", "row", "col", "row", M=128, N=256, K=64, seed=37)
    base = run(p)
    p.bias = syn.cast(np.random.default_rng(38).integers(-3, 4, p.N).astype(np.float32), "f16")
    shifted = run(p)
    want = np.tile(p.bias.to(torch.float64).numpy(), (p.M, 1))
    assert np.array_equal(shifted - base, want)


def test_grouped_same_k_round_robin_integer_exact():
    """Problems that all share K take the static round robin instead of the
    claim queues: 140 problems of K = 96 with M and N from 1 to 384 (more
    tiles than the persistent grid, so workgroups run several), two calls in
    a row, then a mixed-K call on the same plan (queue path) and the same-K
    list again. Every output exact, NaN-prefilled, guards intact."""
    rng = np.random.default_rng(78)
    same = [(int(rng.integers(1, 385)), int(rng.integers(1, 385)), 96) for _ in range(140)]
    mixed = [(64, 200, 8), (300, 64, 1032), (129, 129, 96)]
    plan = g.Plan("f16", la="row", lb="row", lc="row")

    def call(shapes, seed0, what):
        probs = [_int_problem("f16", "f16", "row", "row", "row", M=m, N=n, K=k, seed=seed0 + i)
                 for i, (m, n, k) in enumerate(shapes)]
        ops = [device_operands(p) for p in probs]
        outs = [make_out(p) for p in probs]
        for buf, D in outs:
            D.fill_(float("nan"))
        print(f"[gpu] grouped {what}: {len(probs)} problems", flush=True)
        plan.run_grouped([(p.M, p.N, p.K, o[0], o[1], o[2], d[1])
                          for p, o, d in zip(probs, ops, outs)], 1.0, 1.0)
        torch.cuda.synchronize()
        for p, (buf, D) in zip(probs, outs):
            acceptance.check_exact(logical(D, p), oracle.gemm(p).d_exact, f"{what} {p.M}x{p.N}x{p.K}")
            check_guards(buf, p)

    call(same, 700, "same K, call 0")
    call(same, 700, "same K, call 1")
    call(mixed, 900, "mixed K")
    call(same, 1000, "same K after the queue path")
    plan.close()


def test_prepared_run_matches_run_and_follows_buffer_contents():
    """Plan.prepare checks and packs one run() once: calling it gives run()'s
    result bitwise (exact against the oracle on integer data), sees new
    contents written into the same buffers, and refuses to run once its plan
    is closed."""
    p = _int_problem("f32", "f32", "row", "row", "row", M=128, N=64, K=256, seed=41)
    plan = g.Plan("f32", la="row", lb="row", lc="row")
    A, B, C = (x.to(DEV) for x in (p.A, p.B, p.C))
    D_run = torch.empty_like(C)
    D_prep = torch.full_like(C, float("nan"))
    prep = plan.prepare(A, B, C, D_prep, p.M, p.N, p.K, p.alpha, p.beta)
    for rep in range(2):
        if rep == 1:
            A.mul_(-1.0)   # new contents, same buffer: the oracle's problem follows
            p.A = -p.A
        plan.run(A, B, C, D_run, p.M, p.N, p.K, p.alpha, p.beta)
        D_prep.fill_(float("nan"))
        prep()
        torch.cuda.synchronize()
        assert torch.equal(D_prep, D_run), f"prepared != run (call {rep})"
        exact(D_prep.cpu().numpy().astype(np.float64), p, what=f"prepared call {rep}")
    plan.close()
    with pytest.raises(g.GemmError):
        prep()
