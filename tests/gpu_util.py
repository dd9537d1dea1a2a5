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
