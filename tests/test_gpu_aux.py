"""Auxiliary-tensor epilogue on the GPU against the oracle, through
gemm_plan_run_aux: an M x N tensor X combined by add / sub / mul / div before
or after the activation, and the auxiliary store Z (the activation's input)."""
from __future__ import annotations

import dataclasses
import itertools

import numpy as np
import pytest
import torch

import dense_gemm_epilogue_02_amd as g
import oracle
from oracle import acceptance
import synthetic as syn
from gpu_util import DEV, check_guards, full_size_samples, logical, make_out, scales

pytestmark = pytest.mark.gpu
S, T = g.Schedule, g.Tile
OPS = ("add", "sub", "mul", "div")
POS = ("before", "after")


def run_aux(p, act=None, tile=T.AUTO, schedule=S.AUTO, sk_grid=0, aux_offset=0, store=True,
            in_place=False):
    """Run p (with p.aux, or None) and return (D, Z) as fp64 [M, N] (Z None
    without the store). X goes to the device aux_offset elements into a
    larger buffer (an offset of 1 misaligns it); in_place writes Z over X."""
    plan = g.Plan(p.dtype_ab, p.dtype_cd, p.la, p.lb, p.lc, activation=act)
    plan.set_config(schedule, tile, sk_grid)
    A, B = p.A.to(DEV), p.B.to(DEV)
    C = p.C.to(DEV) if p.C is not None else None
    buf, D = make_out(p)
    X = None
    if p.aux is not None:
        hold = torch.zeros(p.M * p.N + aux_offset, dtype=p.aux.dtype, device=DEV)
        hold[aux_offset:] = p.aux.reshape(-1).to(DEV)
        X = hold[aux_offset:]
    zbuf = Z = None
    if in_place:
        Z = X
    elif store:
        zbuf, Z = make_out(p)
    bias = p.bias.to(DEV) if p.bias is not None else None
    sa, sb = scales(p)
    print(f"[gpu] aux {p.dtype_ab} {p.la}{p.lb}{p.lc} {p.M}x{p.N}x{p.K} op={p.aux_op} "
          f"pos={p.aux_pos} act={act} x={X is not None}+{aux_offset} store={store} "
          f"inplace={in_place} {schedule.name}/{tile.name}", flush=True)
    plan.run_aux(A, B, C, D, p.M, p.N, p.K, aux=X, aux_op=p.aux_op, aux_pos=p.aux_pos,
                 aux_out=Z, alpha=p.alpha, beta=p.beta, scale_a=sa, scale_b=sb, bias=bias)
    torch.cuda.synchronize()
    check_guards(buf, p)
    if zbuf is not None:
        check_guards(zbuf, p)
    plan.close()
    return logical(D, p), (logical(Z, p) if Z is not None else None)


def exact(p, act, what, **kw):
    d, z = run_aux(p, act=act, **kw)
    r = oracle.gemm(p, act=act)
    acceptance.check_exact(d, r.d_exact, what + " D")
    if z is not None:
        acceptance.check_exact(z, r.z_exact, what + " Z")


def close(p, act, what, **kw):
    d, z = run_aux(p, act=act, **kw)
    r = oracle.gemm(p, act=act)
    acceptance.check_close(d, r.ref, r.S, p.dtype_ab, p.dtype_cd, what + " D")
    if z is not None:
        acceptance.check_close(z, r.z_ref, r.z_S, p.dtype_ab, p.dtype_cd, what + " Z")


def int_problem(dtype_ab, dtype_cd, lc="row", M=200, N=136, K=72, seed=120, op="add",
                pos="before", **kw):
    p = syn.integer_problem(M, N, K, dtype_ab=dtype_ab, dtype_cd=dtype_cd, lc=lc, lo=-1, hi=1,
                            with_bias=True, seed=seed, **kw)
    return syn.add_aux(p, op, pos, dist="int_nz" if op == "div" else "int", lo=-3, hi=3,
                       seed=seed + 1)


@pytest.mark.parametrize("op,pos", list(itertools.product(OPS, POS)))
@pytest.mark.parametrize("dtype_ab,dtype_cd", [("f16", "f16"), ("bf16", "bf16"), ("f32", "f32"),
                                               ("f8e4m3", "bf16")])
@pytest.mark.parametrize("lc", ["row", "col"])
def test_aux_integer_exact_ops(op, pos, dtype_ab, dtype_cd, lc):
    """Integer data: every op on both sides of ReLU is exact (a quotient by
    +-1, 2 or 3 never lands on a rounding tie of the output format)."""
    p = int_problem(dtype_ab, dtype_cd, lc=lc, op=op, pos=pos)
    exact(p, "relu", f"{op}/{pos} {dtype_ab} {lc}")


@pytest.mark.parametrize("tile", [T.T256x256, T.T128x128, T.T64x256, T.T32x256, T.GENERIC,
                                  T.WHOLEK])
@pytest.mark.parametrize("la,lb", [("row", "col"), ("row", "row"), ("col", "col")])
def test_aux_integer_exact_tiles(tile, la, lb):
    p = syn.integer_problem(300, 520, 136, dtype_ab="bf16", dtype_cd="bf16", la=la, lb=lb,
                            lo=-1, hi=1, seed=122)
    syn.add_aux(p, "mul", "after", dist="int", lo=-2, hi=2, seed=123)
    exact(p, "relu", f"{tile.name} {la}{lb}", tile=tile, schedule=S.DATA_PARALLEL)


@pytest.mark.parametrize("sched", [S.STREAM_K, S.HYBRID, S.SPLIT_K])
@pytest.mark.parametrize("tile", [T.T256x256, T.T128x128, T.T32x256])
def test_aux_integer_exact_schedules(sched, tile):
    """The partial-tile fixup runs the same epilogue (the last contributor)."""
    p = syn.integer_problem(160, 520, 2048, dtype_ab="f16", dtype_cd="f16", lo=-1, hi=1,
                            seed=124)
    syn.add_aux(p, "sub", "before", dist="int", seed=125)
    exact(p, "relu", f"{sched.name} {tile.name}", tile=tile, schedule=sched, sk_grid=24)


@pytest.mark.parametrize("op,pos", list(itertools.product(OPS, POS)))
@pytest.mark.parametrize("act", ["identity", "sigmoid", "tanh"])
def test_aux_random_close(op, pos, act):
    p = syn.make_problem(384, 520, 264, dtype_ab="bf16", dtype_cd="bf16", dist_c="normal",
                         beta=0.5, dist_bias="normal", seed=126)
    syn.add_aux(p, op, pos, dist="away" if op == "div" else "normal", seed=127)
    close(p, act, f"{op}/{pos}/{act}")


@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_aux_random_close_other_types(dtype):
    p = syn.make_problem(250, 190, 300, dtype_ab=dtype, dtype_cd=dtype, lc="col",
                         dist_c="normal", beta=-1.0, seed=128)
    syn.add_aux(p, "div", "after", dist="away", seed=129)
    close(p, "tanh", dtype)


def test_aux_misaligned_uses_element_epilogue():
    p = int_problem("f16", "f16", M=256, N=256, K=64, op="mul", pos="before", seed=130)
    exact(p, "relu", "aux at +1 element", aux_offset=1)


def test_aux_store_alone_is_the_preactivation():
    p = syn.make_problem(320, 256, 128, dtype_ab="f16", dtype_cd="f16", dist_c="normal",
                         beta=1.0, dist_bias="normal", seed=131)
    p.aux = None
    close(p, "sigmoid", "store only")


def test_aux_without_store():
    p = int_problem("bf16", "bf16", op="add", pos="after", seed=132)
    exact(p, "relu", "no store", store=False)


def test_aux_in_place_store_over_x():
    p = int_problem("f16", "f16", M=256, N=512, K=64, op="mul", pos="before", seed=133)
    exact(p, "relu", "Z over X", in_place=True)


def test_aux_is_c():
    """X may be the same buffer as C."""
    p = int_problem("f16", "f16", M=256, N=256, K=96, op="sub", pos="before", seed=134)
    A, B, C = p.A.to(DEV), p.B.to(DEV), p.C.to(DEV)
    D = torch.empty_like(C)
    plan = g.Plan("f16", "f16", activation="relu")
    plan.run_aux(A, B, C, D, p.M, p.N, p.K, aux=C, aux_op="sub", aux_pos="before",
                 alpha=p.alpha, beta=p.beta, bias=p.bias.to(DEV))
    torch.cuda.synchronize()
    plan.close()
    q = dataclasses.replace(p, aux=p.C)
    acceptance.check_exact(logical(D, q), oracle.gemm(q, act="relu").d_exact, "X = C")


def test_aux_k_zero():
    p = int_problem("bf16", "bf16", M=40, N=48, K=8, op="mul", pos="after", seed=135)
    q = dataclasses.replace(p, K=0, A=p.A[:0], B=p.B[:0])
    exact(q, "relu", "K=0")


@pytest.mark.parametrize("M,N,K", [(4096, 8192, 8192), (4096, 8192, 28672), (16, 8192, 28672)])
def test_aux_full_size_every_block(M, N, K):
    """The residual-add workload's shapes (O and down projections with the
    residual stream as the auxiliary tensor) and a decode row count: every
    output written, one oracle entry in every 32 x 32 block of D and Z plus
    the corners of every tile."""
    p = syn.make_problem(M, N, K, dtype_ab="bf16", dtype_cd="bf16", lb="col", std_b=0.02,
                         seed=136)
    syn.add_aux(p, "add", "before", seed=137)
    d, z = run_aux(p, act="identity")
    plan = g.Plan("bf16", la="row", lb="col", lc="row")
    desc = plan.describe(M, N, K)
    plan.close()
    ii, jj = full_size_samples(M, N, 138, desc)
    r = oracle.gemm_entries(p, ii, jj)
    acceptance.check_close(d[ii, jj], r.ref, r.S, "bf16", "bf16", f"{M}x{N}x{K} D")
    acceptance.check_close(z[ii, jj], r.z_ref, r.z_S, "bf16", "bf16", f"{M}x{N}x{K} Z")
    assert np.isfinite(d).all()
