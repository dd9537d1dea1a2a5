"""Shared helpers of the GPU parity tests: run a synthetic problem through the
C ABI (via the binding) and read D back in logical [M, N] order.

D is written into the middle of a larger buffer whose guard regions hold a
sentinel, so a write outside D is detected; the rest of D starts as NaN so an
element the kernels forget to write fails every comparison.
"""
from __future__ import annotations

import numpy as np
import torch

import dense_gemm_epilogue_02_amd as g
import synthetic as syn

DEV = torch.device("cuda:0")
GUARD = 4096   # elements on each side of D
SENTINEL = 12345.0


def device_operands(p):
    A = p.A.to(DEV)
    B = p.B.to(DEV)
    C = p.C.to(DEV) if p.C is not None else None
    return A, B, C


def make_out(p):
    dt = syn.TORCH_DTYPE[p.dtype_cd]
    buf = torch.full((p.M * p.N + 2 * GUARD,), float("nan"), dtype=dt, device=DEV)
    buf[:GUARD] = SENTINEL
    buf[GUARD + p.M * p.N:] = SENTINEL
    D = buf[GUARD:GUARD + p.M * p.N]
    return buf, D


def check_guards(buf, p):
    sent = torch.tensor(SENTINEL, dtype=buf.dtype).float().item()   # as stored
    head = buf[:GUARD].float().cpu()
    tail = buf[GUARD + p.M * p.N:].float().cpu()
    assert bool((head == sent).all()) and bool((tail == sent).all()), \
        "kernel wrote outside D"


def logical(D, p) -> np.ndarray:
    """fp64 [M, N] view of D (stored in layout p.lc)."""
    d = D.float().cpu().double().numpy()
    if p.lc == "row":
        return d.reshape(p.M, p.N)
    return d.reshape(p.N, p.M).T


def scales(p):
    if p.dtype_ab != "f8e4m3":
        return None, None
    sa = torch.tensor([p.scale_a if p.scale_a is not None else 1.0], dtype=torch.float32,
                      device=DEV)
    sb = torch.tensor([p.scale_b if p.scale_b is not None else 1.0], dtype=torch.float32,
                      device=DEV)
    return sa, sb


def run(p, relu=False, schedule=g.Schedule.AUTO, tile=g.Tile.AUTO, sk_grid=0, plan=None,
        operands=None, in_place=False, act=None, bias_offset=0):
    """Run p on the GPU and return D as fp64 [M, N] (plus the plan's describe()).

    act names the activation (None: ReLU if relu else linear); p.bias, if set,
    goes to the device bias_offset elements into a larger buffer (an offset
    of 1 misaligns it)."""
    own = plan is None
    if own:
        plan = g.Plan(p.dtype_ab, p.dtype_cd, p.la, p.lb, p.lc, relu, activation=act)
    plan.set_config(schedule, tile, sk_grid)
    A, B, C = operands if operands is not None else device_operands(p)
    if in_place:
        buf = None
        D = C
    else:
        buf, D = make_out(p)
    sa, sb = scales(p)
    bias = None
    if getattr(p, "bias", None) is not None:
        hold = torch.zeros(p.N + bias_offset, dtype=p.bias.dtype, device=DEV)
        hold[bias_offset:] = p.bias.to(DEV)
        bias = hold[bias_offset:]
    print(f"[gpu] {p.dtype_ab} {p.la}{p.lb}{p.lc} M={p.M} N={p.N} K={p.K} relu={relu} act={act} "
          f"bias={bias is not None}+{bias_offset} {plan.describe(p.M, p.N, p.K)}", flush=True)
    plan.run(A, B, C, D, p.M, p.N, p.K, p.alpha, p.beta, sa, sb, bias=bias)
    torch.cuda.synchronize()
    if buf is not None:
        check_guards(buf, p)
    out = logical(D, p)
    if own:
        plan.close()
    return out


def block_samples(M, N, seed, block=32):
    """One output entry inside every block x block block of an M x N output
    (a uniformly random position, clipped to the ragged edge), plus the four
    corners of D. 32 x 32 is the MFMA block every tile shape is built from,
    so every tile of every schedule, and every wave's fragment of it, is
    sampled. Returns (ii, jj) index arrays."""
    rng = np.random.default_rng(seed)
    bi = np.arange(0, M, block)
    bj = np.arange(0, N, block)
    I0, J0 = np.meshgrid(bi, bj, indexing="ij")
    hi_i = np.minimum(block, M - I0)
    hi_j = np.minimum(block, N - J0)
    ii = (I0 + (rng.random(I0.shape) * hi_i).astype(np.int64)).ravel()
    jj = (J0 + (rng.random(J0.shape) * hi_j).astype(np.int64)).ravel()
    ii = np.concatenate([ii, [0, 0, M - 1, M - 1]])
    jj = np.concatenate([jj, [0, N - 1, 0, N - 1]])
    return ii, jj


def tile_corner_samples(M, N, bm, bn):
    """The four corners of every bm x bn output tile (the first and last
    rows and columns a tile's waves write)."""
    ti = np.arange(0, M, bm)
    tj = np.arange(0, N, bn)
    rows = np.stack([ti, np.minimum(ti + bm, M) - 1], 1)
    cols = np.stack([tj, np.minimum(tj + bn, N) - 1], 1)
    ii, jj = [], []
    for a in range(2):
        for b in range(2):
            I, J = np.meshgrid(rows[:, a], cols[:, b], indexing="ij")
            ii.append(I.ravel())
            jj.append(J.ravel())
    return np.concatenate(ii), np.concatenate(jj)


def full_size_samples(M, N, seed, describe=None):
    """block_samples plus the corners of every tile of the launch that
    `describe` names (a gemm_plan_describe dict)."""
    ii, jj = block_samples(M, N, seed)
    if describe and describe.get("kernel") == "tile":
        bm, bn = (int(x) for x in describe["tile"].split("x"))
        ci, cj = tile_corner_samples(M, N, bm, bn)
        ii = np.concatenate([ii, ci])
        jj = np.concatenate([jj, cj])
    return ii, jj
