"""gemm_plan_run_noalloc (static workspace, no device allocation) against
gemm_plan_run, through the C ABI: two calls in a row, the second smaller;
bit-exact on integer-valued data, within the fp16/bf16 tolerance of the
oracle on random data; a launch beyond the static workspace is refused."""
import numpy as np
import pytest
import torch

import dense_gemm_epilogue_02_amd as g
import oracle
from oracle import acceptance
import synthetic as syn
from gpu_util import DEV, device_operands, full_size_samples, logical, make_out, check_guards

pytestmark = pytest.mark.gpu
S, T = g.Schedule, g.Tile


def both(p, schedule=S.AUTO, tile=T.AUTO, sk_grid=0):
    """D from gemm_plan_run and from gemm_plan_run_noalloc (one plan each,
    NaN-prefilled, guard regions checked)."""
    outs = []
    for noalloc in (False, True):
        plan = g.Plan(p.dtype_ab, p.dtype_cd, p.la, p.lb, p.lc)
        plan.set_config(schedule, tile, sk_grid)
        A, B, C = device_operands(p)
        buf, D = make_out(p)
        print(f"[gpu] noalloc={noalloc} {p.dtype_ab} {p.la}{p.lb}{p.lc} {p.M}x{p.N}x{p.K} "
              f"{plan.describe(p.M, p.N, p.K)}", flush=True)
        if noalloc:
            g.gemm_plan_run_noalloc(plan.handle, A, B, C, D, p.M, p.N, p.K, p.alpha, p.beta)
        else:
            g.gemm_plan_run(plan.handle, A, B, C, D, p.M, p.N, p.K, p.alpha, p.beta)
        torch.cuda.synchronize()
        check_guards(buf, p)
        outs.append(logical(D, p))
        plan.close()
    return outs


@pytest.mark.parametrize("sched,tile", [(S.AUTO, T.AUTO), (S.STREAM_K, T.T256x256),
                                        (S.SPLIT_K, T.T64x256), (S.HYBRID, T.T256x256)])
def test_noalloc_integer_exact_two_calls(sched, tile):
    # first call: few tiles, long K (stream-K / split-K workspace in use);
    # second call: smaller and ragged
    for (M, N, K, seed) in ((544, 528, 2048, 1), (200, 136, 1032, 2)):
        p = syn.integer_problem(M, N, K, dtype_ab="bf16", dtype_cd="bf16", la="row", lb="col",
                                lc="row", lo=-1, hi=1, beta=1.0, seed=seed)
        ref, got = both(p, sched, tile)
        want = oracle.gemm(p).d_exact
        assert np.isfinite(got).all()
        assert np.array_equal(ref, want), f"gemm_plan_run {M}x{N}x{K}"
        assert np.array_equal(got, want), f"gemm_plan_run_noalloc {M}x{N}x{K} {sched.name}"


def test_noalloc_random_two_calls_capped_hybrid():
    # 272 tiles of 256^2 on 256 workgroups: gemm_plan_run splits the remainder
    # stream-K over the grid; the static workspace holds partials for 64
    # workgroups of 256^2, so the no-allocation call runs it data-parallel
    for (M, N, K, seed) in ((4352, 4096, 1024, 3), (1000, 776, 1032, 4)):
        p = syn.make_problem(M, N, K, dtype_ab="f16", dtype_cd="f16", la="row", lb="col",
                             dist_c="normal", alpha=1.0, beta=0.5, seed=seed)
        ref, got = both(p)
        ii, jj = full_size_samples(M, N, seed)
        r = oracle.gemm_entries(p, ii, jj)
        for d, what in ((ref, "gemm_plan_run"), (got, "gemm_plan_run_noalloc")):
            assert np.isfinite(d).all(), what
            acceptance.check_close(d[ii, jj], r.ref, r.S, "f16", "f16", f"{what} {M}x{N}x{K}")


def test_noalloc_refuses_launch_beyond_static_workspace():
    # stream-K forced over 130 x 130 tiles of 128^2: 16900 arrival counters
    M = N = 128 * 130
    K = 64
    plan = g.Plan("bf16", la="row", lb="col", lc="row")
    plan.set_config(S.STREAM_K, T.T128x128, 0)
    A = torch.zeros(M * K, dtype=torch.bfloat16, device=DEV)
    B = torch.zeros(N * K, dtype=torch.bfloat16, device=DEV)
    D = torch.full((M * N,), 7.0, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(g.GemmError) as ei:
        g.gemm_plan_run_noalloc(plan.handle, A, B, None, D, M, N, K, 1.0, 0.0)
    assert ei.value.status == 2 and "static workspace" in str(ei.value)
    torch.cuda.synchronize()
    assert bool((D == 7.0).all()), "a refused call enqueued work"
    plan.close()
