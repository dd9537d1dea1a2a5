"""MX block-scaled GEMM (e4m3 elements, one E8M0 scale per 32 K elements of
each row of A and column of B) on the GPU against the oracle, through
gemm_plan_run_mx."""
from __future__ import annotations

import itertools

import numpy as np
import pytest
import torch

import dense_gemm_epilogue_02_amd as g
import oracle
from oracle import acceptance
import synthetic as syn
from gpu_util import DEV, check_guards, full_size_samples, logical, make_out

pytestmark = pytest.mark.gpu
S, T = g.Schedule, g.Tile
LAYOUTS = list(itertools.product(("row", "col"), repeat=3))
TILES = [T.AUTO, T.T256x256, T.T128x128, T.T64x256, T.T32x256, T.GENERIC]


def run_mx(p, tile=T.AUTO, schedule=S.AUTO, sk_grid=0, act=None, scale_offset=0):
    """p.mx_a / p.mx_b go to the device scale_offset bytes into larger
    buffers (an offset that is not a multiple of 4 forces the scalar kernel)."""
    plan = g.Plan(p.dtype_ab, "bf16", p.la, p.lb, p.lc, activation=act)
    plan.set_config(schedule, tile, sk_grid)
    A, B = p.A.to(DEV), p.B.to(DEV)
    C = p.C.to(DEV) if p.C is not None else None
    buf, D = make_out(p)

    def dev_scales(x):
        hold = torch.zeros(x.numel() + scale_offset, dtype=torch.uint8, device=DEV)
        hold[scale_offset:] = x.reshape(-1).to(DEV)
        return hold[scale_offset:]

    xa, xb = dev_scales(p.mx_a), dev_scales(p.mx_b)
    bias = p.bias.to(DEV) if p.bias is not None else None
    print(f"[gpu] mx {p.dtype_ab} {p.la}{p.lb}{p.lc} {p.M}x{p.N}x{p.K} {schedule.name}/{tile.name} "
          f"act={act} bias={bias is not None} off={scale_offset}", flush=True)
    plan.run_mx(A, B, C, D, p.M, p.N, p.K, xa, xb, p.alpha, p.beta, bias=bias)
    torch.cuda.synchronize()
    check_guards(buf, p)
    plan.close()
    return logical(D, p)


def exact(got, p, act=None, what=""):
    acceptance.check_exact(got, oracle.gemm(p, act=act).d_exact, what)


def close(got, p, act=None, what=""):
    r = oracle.gemm(p, act=act)
    acceptance.check_close(got, r.ref, r.S, "f8e4m3", "bf16", what)


@pytest.mark.parametrize("la,lb,lc", LAYOUTS)
@pytest.mark.parametrize("tile", TILES)
def test_mx_integer_exact_layouts_tiles(la, lb, lc, tile):
    p = syn.mx_integer_problem(304, 272, 384, la=la, lb=lb, lc=lc, lo=-1, hi=1, seed=90)
    exact(run_mx(p, tile=tile, schedule=S.DATA_PARALLEL), p, what=f"{la}{lb}{lc} {tile.name}")


@pytest.mark.parametrize("sched", [S.STREAM_K, S.HYBRID, S.SPLIT_K])
@pytest.mark.parametrize("tile", [T.T256x256, T.T128x128, T.T64x256, T.T32x256])
def test_mx_integer_exact_schedules(sched, tile):
    p = syn.mx_integer_problem(200, 520, 2048, lo=-1, hi=1, seed=91, with_bias=True)
    exact(run_mx(p, tile=tile, schedule=sched, sk_grid=24, act="relu"), p, act="relu",
          what=f"{sched.name} {tile.name}")


@pytest.mark.parametrize("K", [32, 96, 160, 224])
def test_mx_partial_k_tiles_use_scalar_kernel(K):
    p = syn.mx_integer_problem(72, 136, K, seed=92)
    exact(run_mx(p), p, what=f"K={K}")


def test_mx_unaligned_scale_arrays_use_scalar_kernel():
    p = syn.mx_integer_problem(96, 128, 256, seed=93)
    exact(run_mx(p, scale_offset=1), p, what="scales at +1 byte")


@pytest.mark.parametrize("M,N,K", [(512, 512, 512), (64, 1024, 2048), (1000, 376, 640)])
def test_mx_random_close(M, N, K):
    p = syn.make_mx_problem(M, N, K, dist_c="normal", beta=0.5, seed=94)
    close(run_mx(p), p, what=f"{M}x{N}x{K}")


@pytest.mark.parametrize("act", ["sigmoid", "tanh"])
def test_mx_random_bias_activation_close(act):
    p = syn.make_mx_problem(256, 384, 512, dist_bias="normal", seed=95)
    close(run_mx(p, act=act), p, act=act, what=act)


def test_mx_wide_scale_range_close():
    # block scales 2^-12 .. 2^12: the products of one output span 2^48, so
    # the fp32 sums round (no longer exact); within the fp8 tolerance
    p = syn.mx_integer_problem(128, 256, 512, lo=-1, hi=1, emin=-12, emax=12, with_c=False,
                               seed=96)
    close(run_mx(p), p, what="wide scales")


@pytest.mark.parametrize("M,N,K", [(16, 8192, 28672), (4096, 8192, 8192)])
def test_mx_full_size_sampled(M, N, K):
    p = syn.make_mx_problem(M, N, K, seed=97, std_b=0.02)
    got = run_mx(p)
    assert np.isfinite(got).all()
    plan = g.Plan("f8e4m3", "bf16", "row", "col", "row")
    d = plan.describe(M, N, K)
    plan.close()
    ii, jj = full_size_samples(M, N, 98, d)
    r = oracle.gemm_entries(p, ii, jj)
    acceptance.check_close(got[ii, jj], r.ref, r.S, "f8e4m3", "bf16", f"{M}x{N}x{K} every block")


def test_mx_nan_scale_gives_nan_row_and_column():
    p = syn.mx_integer_problem(64, 64, 256, seed=99, with_c=False)
    p.mx_a[5, 2] = 255
    p.mx_b[9, 7] = 255
    for tile in (T.AUTO, T.GENERIC):
        got = run_mx(p, tile=tile)
        want = np.isnan(oracle.gemm(p).ref)
        assert np.array_equal(np.isnan(got), want), tile.name


def test_mx_k_zero_is_beta_c_plus_bias():
    p = syn.mx_integer_problem(40, 48, 32, seed=100, with_bias=True)
    import dataclasses
    q = dataclasses.replace(p, K=0, A=p.A[:0], B=p.B[:0], mx_a=p.mx_a[:, :0],
                            mx_b=p.mx_b[:, :0])
    exact(run_mx(q), q, what="K=0")


def test_mx_layer_bench_inputs_sampled():
    """The MXFP8 layer benchmark's own inputs (drawn and MX-quantized on the
    device, QKV 4096x10240x8192, seed 0) in its launch; sampled outputs
    against the oracle on the same bytes."""
    M, N, K, A, B, xa, xb = syn.mx_layer_device("qkv", DEV, seed=0)
    plan = g.Plan("f8e4m3", "bf16", "row", "col", "row")
    D = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=DEV)
    print(f"[gpu] mx layer qkv {plan.describe(M, N, K)}", flush=True)
    plan.run_mx(A, B, None, D, M, N, K, xa, xb)
    torch.cuda.synchronize()
    plan.close()
    p = syn.Problem(M, N, K, A.cpu(), B.cpu(), None, 1.0, 0.0, None, None, "f8e4m3", "bf16",
                    "row", "col", "row", None, xa.cpu(), xb.cpu())
    assert bool(torch.isfinite(D).all())
    plan = g.Plan("f8e4m3", "bf16", "row", "col", "row")
    d = plan.describe(M, N, K)
    plan.close()
    ii, jj = full_size_samples(M, N, 101, d)
    r = oracle.gemm_entries(p, ii, jj)
    got = D.float().cpu().double().numpy()[ii, jj]
    acceptance.check_close(got, r.ref, r.S, "f8e4m3", "bf16", "mx layer qkv every block")


# ------------------------------------------------------------ MXFP4
# "Generating State-of-the-Art GEMMs with TorchInductor's CuteDSL backend",
# section 5.1: MXF4 beside MXFP8 in the scaled mm family. e2m1 elements, two
# per byte along K for the tile kernels (A RowMajor, B ColumnMajor).

F4 = "f4e2m1"


@pytest.mark.parametrize("tile", [T.T256x256, T.T128x128, T.T64x256, T.T32x256, T.GENERIC])
@pytest.mark.parametrize("lc", ["row", "col"])
def test_mxfp4_integer_exact_tiles(tile, lc):
    # ragged M and N, K = 768: three k-tiles of 256 elements
    p = syn.mx_integer_problem(304, 272, 768, lc=lc, lo=-4, hi=4, seed=120, elem=F4)
    exact(run_mx(p, tile=tile, schedule=S.DATA_PARALLEL), p, what=f"mxfp4 {tile.name} lc={lc}")


@pytest.mark.parametrize("sched,tile", [(S.STREAM_K, T.T256x256), (S.STREAM_K, T.T128x128),
                                        (S.HYBRID, T.T128x128), (S.SPLIT_K, T.T64x256),
                                        (S.SPLIT_K, T.T32x256), (S.AUTO, T.AUTO)])
def test_mxfp4_integer_exact_schedules(sched, tile):
    p = syn.mx_integer_problem(200, 264, 4096, lo=-2, hi=2, seed=121, elem=F4)
    exact(run_mx(p, tile=tile, schedule=sched, sk_grid=37 if sched == S.STREAM_K else 0), p,
          what=f"mxfp4 {sched.name} {tile.name}")


@pytest.mark.parametrize("la,lb", [("row", "row"), ("col", "col"), ("col", "row")])
def test_mxfp4_other_layouts_on_scalar_kernel(la, lb):
    # packed along each operand's contiguous dimension: no tile kernel, the
    # scalar kernel reads the nibbles
    p = syn.mx_integer_problem(48, 40, 256, la=la, lb=lb, lo=-4, hi=4, seed=122, elem=F4)
    plan = g.Plan(F4, "bf16", la, lb, "row")
    assert plan.describe(p.M, p.N, p.K)["kernel"] == "generic"
    plan.close()
    exact(run_mx(p), p, what=f"mxfp4 {la}{lb}")


@pytest.mark.parametrize("K", [32, 96, 288])
def test_mxfp4_partial_k_tiles_use_scalar_kernel(K):
    p = syn.mx_integer_problem(64, 128, K, lo=-4, hi=4, seed=123, elem=F4)
    exact(run_mx(p), p, what=f"mxfp4 K={K}")


@pytest.mark.parametrize("M,N,K", [(512, 512, 512), (64, 1024, 2048), (1000, 376, 1280)])
def test_mxfp4_random_close(M, N, K):
    p = syn.make_mx_problem(M, N, K, dist_c="normal", beta=0.5, seed=124, elem=F4)
    got = run_mx(p, act="relu")
    close(got, p, act="relu", what=f"mxfp4 {M}x{N}x{K}")


def test_mxfp4_equals_mxfp8_of_the_same_values_on_gpu():
    # the FP4 kernels against the FP8 kernels on the same element values and
    # scales: identical outputs (both sums exact in fp32 here)
    import dataclasses
    q4 = syn.mx_integer_problem(256, 512, 1024, lo=-4, hi=4, seed=125, elem=F4)
    codes_a = syn.unpack_e2m1(syn.raw(q4.A))
    codes_b = syn.unpack_e2m1(syn.raw(q4.B))
    vals = oracle.decode("f4e2m1", np.arange(16, dtype=np.uint32))
    q8 = dataclasses.replace(q4, A=syn.cast(vals[codes_a].astype(np.float32), "f8e4m3"),
                             B=syn.cast(vals[codes_b].astype(np.float32), "f8e4m3"),
                             dtype_ab="f8e4m3")
    assert np.array_equal(run_mx(q4), run_mx(q8))


def test_mxfp4_full_size_every_block():
    # the MXFP4 layer shape the benchmark times (O projection 4096 x 8192 x 8192)
    p = syn.make_mx_problem(4096, 8192, 8192, seed=126, std_b=0.02, elem=F4)
    got = run_mx(p)
    assert np.isfinite(got).all()
    plan = g.Plan(F4, "bf16", "row", "col", "row")
    d = plan.describe(p.M, p.N, p.K)
    plan.close()
    assert d["kernel"] == "tile"
    ii, jj = full_size_samples(p.M, p.N, 127, d)
    r = oracle.gemm_entries(p, ii, jj)
    acceptance.check_close(got[ii, jj], r.ref, r.S, F4, "bf16", "mxfp4 4096x8192x8192 every block")


def test_mxfp4_plan_refuses_unscaled_runs():
    plan = g.Plan(F4, "bf16", "row", "col", "row")
    A = torch.zeros(64 * 32, dtype=torch.uint8, device=DEV)
    B = torch.zeros(64 * 32, dtype=torch.uint8, device=DEV)
    D = torch.empty(64 * 64, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(g.GemmError) as ei:
        plan.run(A, B, None, D, 64, 64, 64)
    assert ei.value.status == g.Status.UNSUPPORTED and "MX" in str(ei.value)
    plan.close()
