"""Runs captured into a HIP graph (through torch.cuda.graph) and replayed.

Callers that capture their launches need every call of the library to be
capturable once the plan is warm: no allocation, no memset node, no host
wait. Each case runs eagerly once (that call may size the plan's
workspace), captures one call, then replays the graph three times with
other eager GEMMs on the same plan in between, and compares every replay
with the eager result bitwise (NaN-prefilled D before each replay). Cases:
the whole-K kernel, a data-parallel tile launch, a stream-K launch and a
split-K launch (their arrival counters reset themselves in the kernel), and
the no-allocation entry point on a stream-K launch.
"""
import pytest
import torch

import dense_gemm_epilogue_02_amd as g
import synthetic as syn
from gpu_util import device_operands, make_out

pytestmark = pytest.mark.gpu
S, T = g.Schedule, g.Tile

CASES = [
    ("wholek", "f16", 200, 136, 512, S.AUTO, T.WHOLEK, False),
    ("tile_dp", "bf16", 1024, 768, 512, S.DATA_PARALLEL, T.T128x128, False),
    ("stream_k", "bf16", 544, 528, 2048, S.STREAM_K, T.T256x256, False),
    ("split_k", "f16", 200, 272, 2064, S.SPLIT_K, T.T64x256, False),
    ("noalloc_stream_k", "bf16", 544, 528, 2048, S.STREAM_K, T.T128x128, True),
]


@pytest.mark.parametrize("name,dt,M,N,K,sched,tile,noalloc", CASES, ids=[c[0] for c in CASES])
def test_graph_replay_matches_eager(name, dt, M, N, K, sched, tile, noalloc):
    seed = 300 + 2 * [c[0] for c in CASES].index(name)
    p = syn.make_problem(M, N, K, dtype_ab=dt, dtype_cd=dt, la="row", lb="col", lc="row",
                         dist_c="normal", alpha=1.0, beta=0.5, seed=seed)
    other = syn.make_problem(M, N, K, dtype_ab=dt, dtype_cd=dt, la="row", lb="col", lc="row",
                             dist_c="normal", alpha=1.0, beta=0.5, seed=seed + 1)
    plan = g.Plan(dt, la="row", lb="col", lc="row")
    plan.set_config(sched, tile, 0)
    print(f"[gpu] graph {name} {plan.describe(M, N, K)}", flush=True)
    A, B, C = device_operands(p)
    _, D = make_out(p)
    A2, B2, C2 = device_operands(other)
    _, D2 = make_out(other)

    def call(a, b, c, d):
        if noalloc:
            g.gemm_plan_run_noalloc(plan.handle, a, b, c, d, M, N, K, 1.0, 0.5)
        else:
            plan.run(a, b, c, d, M, N, K, 1.0, 0.5)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(A, B, C, D)                       # eager: sizes the workspace
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    eager = D.clone()
    assert bool(torch.isfinite(eager).all())

    graph = torch.cuda.CUDAGraph()
    D.fill_(float("nan"))
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        call(A, B, C, D)
    torch.cuda.synchronize()
    for rep in range(3):
        call(A2, B2, C2, D2)                   # other eager work on the same plan
        D.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(D, eager), f"{name}: replay {rep} differs from the eager run"
    plan.close()
