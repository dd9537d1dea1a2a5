"""Batched GEMM on the GPU against the oracle: gemm_plan_run_batched runs
batch_count problems of one shape from strided operands in one launch.

Each batch entry is its own seeded problem; the test packs the entries into
strided device buffers (gaps between entries hold a sentinel, so a write
outside an entry's D is caught) and compares every entry with the oracle.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import pytest
import torch

import dense_gemm_epilogue_02_amd as g
import oracle
from oracle import acceptance
import synthetic as syn
from gpu_util import DEV, SENTINEL, full_size_samples, logical, scales

pytestmark = pytest.mark.gpu
S, T = g.Schedule, g.Tile
FAMS = [("f32", "f32"), ("f16", "f16"), ("bf16", "bf16"), ("f8e4m3", "bf16")]
_BITS = {1: torch.uint8, 2: torch.int16, 4: torch.int32}


def _bits(t):
    return t.view(_BITS[t.element_size()])


def pack(tensors, stride, dtype, fill=None):
    """Device buffer holding tensors[b] at element offset b*stride (stride 0:
    one shared copy); the rest is `fill` (zero bits when None)."""
    n = tensors[0].numel()
    total = (len(tensors) - 1) * stride + n
    buf = torch.zeros(max(total, 1), dtype=dtype, device=DEV)
    if fill is not None:
        buf.fill_(fill)
    raw = _bits(buf)
    for b, t in enumerate(tensors):
        if stride == 0 and b > 0:
            break
        raw[b * stride:b * stride + n] = _bits(t.reshape(-1)).to(DEV)
    return buf


def share(probs, *names):
    """Make every entry use entry 0's operands `names` (a stride-0 operand)."""
    return [dataclasses.replace(p, **{n: getattr(probs[0], n) for n in names}) for p in probs]


def run_batched(probs, strides, relu=False, act=None, schedule=S.AUTO, tile=T.AUTO, sk_grid=0):
    """Run the entries through one gemm_plan_run_batched call; return each
    entry's D as fp64 [M, N] after checking the sentinel gaps."""
    p0 = probs[0]
    M, N, K, nb = p0.M, p0.N, p0.K, len(probs)
    sa, sb, sc, sd = strides
    assert sd >= M * N
    dab, dcd = syn.TORCH_DTYPE[p0.dtype_ab], syn.TORCH_DTYPE[p0.dtype_cd]
    A = pack([p.A for p in probs], sa, dab)
    B = pack([p.B for p in probs], sb, dab)
    C = pack([p.C for p in probs], sc, dcd) if p0.C is not None else None
    Dbuf = torch.full(((nb - 1) * sd + M * N,), SENTINEL, dtype=dcd, device=DEV)
    for b in range(nb):
        Dbuf[b * sd:b * sd + M * N] = float("nan")
    bias = p0.bias.to(DEV) if p0.bias is not None else None
    s_a, s_b = scales(p0)
    plan = g.Plan(p0.dtype_ab, p0.dtype_cd, p0.la, p0.lb, p0.lc, relu, activation=act)
    plan.set_config(schedule, tile, sk_grid)
    print(f"[gpu] batched {p0.dtype_ab} {p0.la}{p0.lb}{p0.lc} {M}x{N}x{K} x{nb} strides={strides} "
          f"act={act or ('relu' if relu else 'linear')} bias={bias is not None} "
          f"{schedule.name}/{tile.name}", flush=True)
    plan.run_batched(A, B, C, Dbuf, M, N, K, nb, strides, p0.alpha, p0.beta, s_a, s_b,
                     bias=bias)
    torch.cuda.synchronize()
    plan.close()
    host = Dbuf.float().cpu()
    sent = torch.tensor(SENTINEL, dtype=dcd).float().item()
    outs = []
    for b in range(nb):
        lo, hi = b * sd, b * sd + M * N
        if b + 1 < nb:
            assert bool((host[hi:(b + 1) * sd] == sent).all()), f"write into the gap after entry {b}"
        outs.append(logical(Dbuf[lo:hi], p0))
    return outs


def _int_entries(dab, dcd, la="row", lb="col", lc="row", M=200, N=272, K=208, nb=3,
                 with_bias=False, beta=1.0):
    lo, hi = (-1, 1) if dcd == "bf16" else (-2, 2)
    probs = [syn.integer_problem(M, N, K, dtype_ab=dab, dtype_cd=dcd, la=la, lb=lb, lc=lc,
                                 lo=lo, hi=hi, beta=beta, with_bias=with_bias, seed=40 + b)
             for b in range(nb)]
    return share(probs, "bias") if with_bias else probs


def _packed(p, gap=(0, 0, 0, 0)):
    """Strides of back-to-back entries plus gaps (in elements)."""
    return (p.M * p.K + gap[0], p.K * p.N + gap[1], p.M * p.N + gap[2], p.M * p.N + gap[3])


def exact_all(outs, probs, relu=False, act=None, what=""):
    for b, (got, r) in enumerate(zip(outs, oracle.batched(probs, relu=relu, act=act))):
        acceptance.check_exact(got, r.d_exact, f"{what} entry {b}")


def close_all(outs, probs, relu=False, act=None, what=""):
    for b, (got, r) in enumerate(zip(outs, oracle.batched(probs, relu=relu, act=act))):
        acceptance.check_close(got, r.ref, r.S, probs[0].dtype_ab, probs[0].dtype_cd,
                               f"{what} entry {b}")


@pytest.mark.parametrize("dab,dcd", FAMS)
@pytest.mark.parametrize("tile", [T.AUTO, T.T256x256, T.T128x128, T.T64x256, T.T32x256,
                                  T.GENERIC])
def test_batched_integer_exact_tiles(dab, dcd, tile):
    probs = _int_entries(dab, dcd)
    # gaps of 16 elements keep every entry 16-byte aligned for any element size
    outs = run_batched(probs, _packed(probs[0], (16, 32, 16, 16)), tile=tile,
                       schedule=S.DATA_PARALLEL)
    exact_all(outs, probs, what=f"{dab} {tile.name}")


@pytest.mark.parametrize("la,lb,lc", [("row", "row", "row"), ("col", "col", "col"),
                                      ("row", "col", "col"), ("col", "row", "row")])
@pytest.mark.parametrize("sched", [S.AUTO, S.STREAM_K, S.HYBRID, S.SPLIT_K])
def test_batched_integer_exact_layouts_schedules(la, lb, lc, sched):
    probs = _int_entries("bf16", "bf16", la, lb, lc, M=136, N=264, K=1040, nb=4,
                         with_bias=True)
    outs = run_batched(probs, _packed(probs[0]), relu=True, schedule=sched, sk_grid=24)
    exact_all(outs, probs, relu=True, what=f"{la}{lb}{lc} {sched.name}")


@pytest.mark.parametrize("shared", [("B",), ("A",), ("B", "C")])
def test_batched_stride_zero_shares_operand(shared):
    probs = share(_int_entries("f16", "f16", nb=5), *shared)
    st = list(_packed(probs[0]))
    for n in shared:
        st["ABC".index(n)] = 0
    outs = run_batched(probs, tuple(st))
    exact_all(outs, probs, what=f"shared {shared}")


def test_batched_unaligned_strides_run_entry_by_entry():
    # A stride of M*K + 1 fp16 elements breaks 16-byte alignment of every
    # other entry: the library launches entries one at a time (and the
    # misaligned ones take the scalar kernel) with the same results
    probs = _int_entries("f16", "f16", M=64, N=128, K=96, nb=4)
    outs = run_batched(probs, _packed(probs[0], (1, 0, 3, 5)))
    exact_all(outs, probs, what="unaligned strides")


def test_batched_random_fp8_bias_activation_close():
    rng = np.random.default_rng(70)
    probs = [syn.make_problem(96, 512, 1024, dtype_ab="f8e4m3", dtype_cd="bf16", la="row",
                              lb="col", dist_bias="normal", rng=rng) for _ in range(3)]
    # per-tensor scales and the bias are shared by the batch: every entry
    # takes entry 0's (the oracle is told the same)
    probs = [dataclasses.replace(p, scale_a=probs[0].scale_a, scale_b=probs[0].scale_b,
                                 bias=probs[0].bias) for p in probs]
    outs = run_batched(probs, _packed(probs[0]), act="tanh")
    close_all(outs, probs, act="tanh", what="fp8 tanh")


def test_batched_equals_loop_of_single_runs_bitwise():
    rng = np.random.default_rng(71)
    probs = [syn.make_problem(320, 384, 512, dtype_ab="bf16", dtype_cd="bf16", dist_c="normal",
                              beta=0.5, rng=rng) for _ in range(3)]
    outs = run_batched(probs, _packed(probs[0]), schedule=S.DATA_PARALLEL, tile=T.T128x128)
    from gpu_util import run
    for b, p in enumerate(probs):
        single = run(p, schedule=S.DATA_PARALLEL, tile=T.T128x128)
        assert np.array_equal(outs[b], single), f"entry {b} differs from a single run"
    close_all(outs, probs, what="bf16 random")


def test_batched_count_zero_and_one():
    probs = _int_entries("bf16", "bf16", M=64, N=64, K=64, nb=1)
    exact_all(run_batched(probs, _packed(probs[0])), probs, what="batch 1")
    plan = g.Plan("bf16")
    plan.run_batched(None, None, None, None, 64, 64, 64, 0, (0, 0, 0, 4096))
    plan.close()


def test_batched_in_place_sixteen_entries():
    # the batched example on the CUTLASS Python page: 16 fp16 entries with
    # N(0,1) A and B, C = 0, D written over C, strides M*K, K*N, M*N
    rng = np.random.default_rng(72)
    M, N, K, nb = 256, 128, 192, 16
    probs = [syn.make_problem(M, N, K, dtype_ab="f16", dtype_cd="f16", dist_c="zeros",
                              rng=rng) for _ in range(nb)]
    A = pack([p.A for p in probs], M * K, torch.float16)
    B = pack([p.B for p in probs], K * N, torch.float16)
    C = pack([p.C for p in probs], M * N, torch.float16)
    plan = g.Plan("f16")
    print(f"[gpu] batched in place {M}x{N}x{K} x{nb}", flush=True)
    plan.run_batched(A, B, C, C, M, N, K, nb, (M * K, K * N, M * N, M * N), 1.0, 0.0)
    torch.cuda.synchronize()
    plan.close()
    outs = [logical(C[b * M * N:(b + 1) * M * N], probs[0]) for b in range(nb)]
    close_all(outs, probs, what="in place x16")


def test_batched16_fp16_1024_full_size_every_block():
    """The benchmark's batched configuration (16 x fp16 1024^3, strides M*K,
    K*N, 0, M*N, beta 0, the same seeds), in the launch bench.py times: every
    entry fully written, and one oracle entry in every 32 x 32 block of every
    entry plus the corners of every tile."""
    M = N = K = 1024
    nb = 16
    probs = [syn.make_problem(M, N, K, dtype_ab="f16", dtype_cd="f16", seed=200 + b)
             for b in range(nb)]
    A = torch.stack([q.A for q in probs]).to(DEV)
    B = torch.stack([q.B for q in probs]).to(DEV)
    D = torch.full((nb, M, N), float("nan"), dtype=torch.float16, device=DEV)
    plan = g.Plan("f16", la="row", lb="row", lc="row")
    d = plan.describe_batched(M, N, K, nb)
    print(f"[gpu] batched16 full size {d}", flush=True)
    plan.run_batched(A, B, None, D, M, N, K, nb, (M * K, K * N, 0, M * N))
    torch.cuda.synchronize()
    plan.close()
    assert bool(torch.isfinite(D).all())
    for b in range(nb):
        ii, jj = full_size_samples(M, N, 73 + b, d)
        r = oracle.gemm_entries(probs[b], ii, jj)
        got = D[b].float().cpu().double().numpy()[ii, jj]
        acceptance.check_close(got, r.ref, r.S, "f16", "f16", f"batched16 entry {b}")
