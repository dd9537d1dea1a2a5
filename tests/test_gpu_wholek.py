"""GPU parity of the whole-K kernel (GEMM_TILE_WHOLEK) against the CPU oracle.

Each workgroup owns a 32x32 block of D and its four waves load a quarter of K
each, all at once (fp32 beyond K = 512: eight waves of an eighth); it takes
problems with K <= 1024. Bars as elsewhere: bit-exact on integer-valued data,
the oracle's tolerances otherwise. Every case first checks (host-only
describe) that the launch really is the whole-K kernel, so a silent fallback
to the tile kernels cannot pass for it.
"""
import itertools

import pytest

import dense_gemm_epilogue_02_amd as g
import oracle
from oracle import acceptance
import synthetic as syn
from gpu_util import run

pytestmark = pytest.mark.gpu

S, T = g.Schedule, g.Tile
FAMS = [("f32", "f32"), ("f16", "f16"), ("bf16", "bf16")]
LAYOUTS = list(itertools.product(("row", "col"), repeat=3))


def _int(dab, dcd, la="row", lb="row", lc="row", M=75, N=97, K=200, seed=0, **kw):
    lo, hi = (-1, 1) if dcd == "bf16" else (-2, 2)
    return syn.integer_problem(M, N, K, dtype_ab=dab, dtype_cd=dcd, la=la, lb=lb, lc=lc,
                               lo=lo, hi=hi, seed=seed, **kw)


def _is_wholek(p, relu=False):
    plan = g.Plan(p.dtype_ab, p.dtype_cd, p.la, p.lb, p.lc, relu)
    try:
        plan.set_config(S.AUTO, T.WHOLEK, 0)
        d = plan.describe(p.M, p.N, p.K)
    finally:
        plan.close()
    assert d["kernel"] == "wholek", d
    return d


def _exact(p, relu=False, what=""):
    _is_wholek(p, relu)
    got = run(p, relu=relu, tile=T.WHOLEK)
    acceptance.check_exact(got, oracle.gemm(p, relu=relu).d_exact, what)


@pytest.mark.parametrize("dab,dcd", FAMS)
@pytest.mark.parametrize("la,lb,lc", LAYOUTS)
def test_wholek_integer_exact_all_layouts(dab, dcd, la, lb, lc):
    # M, N not multiples of 32; K not a multiple of a wave's range
    _exact(_int(dab, dcd, la, lb, lc), what=f"{dab} {la}{lb}{lc}")


@pytest.mark.parametrize("dab,dcd", FAMS)
def test_wholek_k_extents(dab, dcd):
    # K = 8: one step, three waves past K; 40: waves ending mid-range; 512
    # and 1024 - 8, 1024: 16 steps per wave (fp32: four, then eight waves)
    for K in (8, 40, 504, 512, 520, 1016, 1024):
        _exact(_int(dab, dcd, M=33, N=64, K=K, seed=K), what=f"{dab} K={K}")


@pytest.mark.parametrize("dab,dcd", FAMS)
def test_wholek_any_k_when_mn_contiguous(dab, dcd):
    # M-contiguous A and N-contiguous B load element by element: no K
    # alignment needed
    for K in (1, 13, 99):
        _exact(_int(dab, dcd, la="col", lb="row", M=40, N=31, K=K, seed=K), what=f"{dab} K={K}")


@pytest.mark.parametrize("dab,dcd", FAMS)
def test_wholek_single_element_and_tiny(dab, dcd):
    for M, N in ((1, 1), (1, 70), (70, 1), (32, 32)):
        _exact(_int(dab, dcd, la="row", lb="col", M=M, N=N, K=16, seed=M + N), what=f"{M}x{N}")


@pytest.mark.parametrize("dab,dcd", FAMS)
@pytest.mark.parametrize("lc", ["row", "col"])
def test_wholek_epilogue_integer_exact(dab, dcd, lc):
    # alpha = 2, beta = -1 with C, a bias row, ReLU
    p = _int(dab, dcd, lc=lc, M=66, N=90, K=64, alpha=2.0, beta=-1.0, with_bias=True, seed=3)
    _exact(p, relu=True, what=f"{dab} epilogue lc={lc}")


def test_wholek_config1_fp32_small_tolerance():
    p = syn.config1()
    d = _is_wholek(p)
    assert d["grid"] == 8
    r = oracle.gemm(p)
    acceptance.check_close(run(p, tile=T.WHOLEK), r.ref, r.S, p.dtype_ab, p.dtype_cd,
                           "fp32 128x64x256 whole-K")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_wholek_random_tolerance(dtype):
    p = syn.make_problem(200, 136, 1000, dtype_ab=dtype, dtype_cd=dtype, la="row", lb="row",
                         lc="row", dist_c="normal", alpha=0.75, beta=-0.5, seed=9)
    _is_wholek(p, relu=True)
    r = oracle.gemm(p, relu=True)
    acceptance.check_close(run(p, relu=True, tile=T.WHOLEK), r.ref, r.S, p.dtype_ab, p.dtype_cd,
                           f"{dtype} 200x136x1000 whole-K")


def test_wholek_fp32_eight_waves_ones_closed_form():
    # the all-ones 1024^3 fp32 problem: D = K + 1 everywhere
    p = syn.config1_ones(1024, "f32")
    d = _is_wholek(p)
    assert d["waves"] == 8
    assert (run(p, tile=T.WHOLEK) == 1025.0).all()


def test_wholek_deterministic():
    p = syn.make_problem(96, 80, 512, dtype_ab="f32", dtype_cd="f32", dist_c="normal", seed=4)
    a = run(p, tile=T.WHOLEK)
    b = run(p, tile=T.WHOLEK)
    assert (a == b).all()


def test_wholek_falls_back_when_it_cannot_take_the_problem():
    # K = 1040 is past its reach; K-contiguous fp16 rows of 13 elements are
    # not 16-byte rows: both run on the other kernels, still exact
    for p in (_int("f32", "f32", K=1040), _int("f16", "f16", la="row", lb="col", K=13)):
        plan = g.Plan(p.dtype_ab, p.dtype_cd, p.la, p.lb, p.lc)
        plan.set_config(S.AUTO, T.WHOLEK, 0)
        d = plan.describe(p.M, p.N, p.K)
        plan.close()
        assert d["kernel"] != "wholek", d
        got = run(p, tile=T.WHOLEK)
        acceptance.check_exact(got, oracle.gemm(p).d_exact, f"fallback K={p.K}")
