"""Seeded synthetic inputs for the GEMM D = alpha*A*B + beta*C.

This module is shared by the CPU oracle side and the HIP side. It holds
random draws and storage-format casts only -- none of the GEMM arithmetic.

Draws follow the distributions the pages use for their examples:
``torch.rand`` (U[0,1)) in the CUTLASS Python walkthrough ("CUTLASS Python
接口全解析", section 2.1, fp32 128x256 @ 256x64 with C = 0) and ``torch.randn``
(N(0,1)) in the CUTLASS Python blog ("CUTLASS Python接口", section 3.3,
fp16 1024^3). Weight-like operands use N(0, 0.02^2).

Every array is drawn in fp32 with ``numpy.random.default_rng(seed)`` in a
fixed order (A, then B, then C of each problem) and then cast once, with
round-to-nearest-even, to the storage type. fp8 operands are quantized per
tensor: s = max|X| / 448 (fp32), X_q = e4m3fn(clamp(X / s, -448, 448)).

Each generator returns CPU torch tensors in *storage layout*: a RowMajor
R x C operand is a contiguous [R, C] tensor; a ColumnMajor one is a
contiguous [C, R] tensor (its transpose). Move them to the GPU with
``.to(device)``; hand their bytes to the oracle with :func:`raw`.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import numpy as np
import torch

# dtype names used across the repository (they match the C enum names)
F32, F16, BF16, F8, F4 = "f32", "f16", "bf16", "f8e4m3", "f4e2m1"
ROW, COL = "row", "col"

# F4 operands are packed two per byte (uint8 storage, see pack_e2m1)
TORCH_DTYPE = {F32: torch.float32, F16: torch.float16, BF16: torch.bfloat16,
               F8: torch.float8_e4m3fn, F4: torch.uint8}
ELEM_BYTES = {F32: 4, F16: 2, BF16: 2, F8: 1}
E4M3_MAX = 448.0
# OCP FP4 E2M1 magnitudes by 3-bit code (exponent bits, fraction bit)
E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
E2M1_MAX = 6.0


def cast(x32: np.ndarray, dtype: str) -> torch.Tensor:
    """RNE cast of an fp32 numpy array to the storage dtype (CPU tensor)."""
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32))
    if dtype == F8:
        t = t.clamp(-E4M3_MAX, E4M3_MAX)
    return t.to(TORCH_DTYPE[dtype])


def raw(t: torch.Tensor) -> np.ndarray:
    """The storage bits of a CPU tensor as a numpy array (no copy when possible)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.float32:
        return t.numpy()
    if t.dtype in (torch.float16, torch.bfloat16):
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    if t.dtype == torch.uint8:          # E8M0 scale codes
        return t.numpy()
    raise TypeError(f"unsupported dtype {t.dtype}")


def to_storage(x32: np.ndarray, layout: str) -> np.ndarray:
    """Logical [R, C] array -> contiguous storage array for ``layout``."""
    return np.ascontiguousarray(x32 if layout == ROW else x32.T)


@dataclass
class Problem:
    """One GEMM's operands in storage layout plus its scalars."""
    M: int
    N: int
    K: int
    A: torch.Tensor
    B: torch.Tensor
    C: Optional[torch.Tensor]
    alpha: float = 1.0
    beta: float = 0.0
    scale_a: Optional[float] = None   # fp8 per-tensor scales (fp32 values)
    scale_b: Optional[float] = None
    dtype_ab: str = BF16
    dtype_cd: str = BF16
    la: str = ROW
    lb: str = ROW
    lc: str = ROW
    bias: Optional[torch.Tensor] = None   # length-N row vector in dtype_cd (None: no bias)
    # MX block scales (E8M0 codes, uint8): mx_a [M, K/32] for the rows of A,
    # mx_b [N, K/32] for the columns of B; None for a non-MX problem
    mx_a: Optional[torch.Tensor] = None
    mx_b: Optional[torch.Tensor] = None
    # auxiliary M x N tensor of the epilogue (dtype_cd, layout lc), its
    # elementwise op ("add", "sub", "mul", "div") and side of the activation
    # ("before", "after"); None: no auxiliary tensor
    aux: Optional[torch.Tensor] = None
    aux_op: str = "add"
    aux_pos: str = "before"

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K


def _draw(rng, shape, dist: str, std: float = 1.0) -> np.ndarray:
    if dist == "uniform":
        return rng.random(shape, dtype=np.float32)
    if dist == "normal":
        x = rng.standard_normal(shape, dtype=np.float32)
        return x if std == 1.0 else (x * np.float32(std)).astype(np.float32)
    if dist == "ones":
        return np.ones(shape, dtype=np.float32)
    if dist == "zeros":
        return np.zeros(shape, dtype=np.float32)
    raise ValueError(dist)


def quantize_e4m3(x32: np.ndarray) -> Tuple[torch.Tensor, float]:
    """Per-tensor fp8 quantization of an fp32 array: (X_q, s) with X ~ s * X_q."""
    amax = float(np.max(np.abs(x32))) if x32.size else 0.0
    s = np.float32(amax / E4M3_MAX) if amax > 0 else np.float32(1.0)
    q = cast((x32 / s).astype(np.float32), F8)
    return q, float(s)


def make_problem(M: int, N: int, K: int, *, dtype_ab: str, dtype_cd: str,
                 la: str = ROW, lb: str = ROW, lc: str = ROW,
                 dist_a: str = "normal", dist_b: str = "normal",
                 dist_c: Optional[str] = None, std_b: float = 1.0,
                 alpha: float = 1.0, beta: float = 0.0,
                 dist_bias: Optional[str] = None,
                 seed: int = 0, rng=None) -> Problem:
    """Draw A (M x K), B (K x N), then C (M x N) if ``dist_c`` is given and a
    length-N bias if ``dist_bias`` is given (in that order)."""
    rng = np.random.default_rng(seed) if rng is None else rng
    a32 = _draw(rng, (M, K), dist_a)
    b32 = _draw(rng, (K, N), dist_b, std_b)
    c = None
    if dist_c is not None:
        c32 = _draw(rng, (M, N), dist_c)
        c = cast(to_storage(c32, lc), dtype_cd)
    bias = None
    if dist_bias is not None:
        bias = cast(_draw(rng, (N,), dist_bias), dtype_cd)
    sa = sb = None
    if dtype_ab == F8:
        A, sa = quantize_e4m3(to_storage(a32, la))
        B, sb = quantize_e4m3(to_storage(b32, lb))
    else:
        A = cast(to_storage(a32, la), dtype_ab)
        B = cast(to_storage(b32, lb), dtype_ab)
    return Problem(M, N, K, A, B, c, alpha, beta, sa, sb, dtype_ab, dtype_cd,
                   la, lb, lc, bias)


def integer_problem(M: int, N: int, K: int, *, dtype_ab: str, dtype_cd: str,
                    la: str = ROW, lb: str = ROW, lc: str = ROW,
                    lo: int = -2, hi: int = 2, beta: float = 1.0,
                    alpha: float = 1.0, with_c: bool = True,
                    with_bias: bool = False, seed: int = 0) -> Problem:
    """Integer-valued operands in [lo, hi] (exact in every storage type)."""
    rng = np.random.default_rng(seed)
    a32 = rng.integers(lo, hi + 1, size=(M, K)).astype(np.float32)
    b32 = rng.integers(lo, hi + 1, size=(K, N)).astype(np.float32)
    c = None
    if with_c:
        c32 = rng.integers(lo, hi + 1, size=(M, N)).astype(np.float32)
        c = cast(to_storage(c32, lc), dtype_cd)
    bias = None
    if with_bias:
        bias = cast(rng.integers(lo, hi + 1, size=(N,)).astype(np.float32), dtype_cd)
    A = cast(to_storage(a32, la), dtype_ab)
    B = cast(to_storage(b32, lb), dtype_ab)
    sa = sb = (1.0 if dtype_ab == F8 else None)
    return Problem(M, N, K, A, B, c, alpha, beta if with_c else 0.0, sa, sb,
                   dtype_ab, dtype_cd, la, lb, lc, bias)


# ---------------------------------------------------------------------------
# The five workloads (shapes and distributions of the pages' examples)
# ---------------------------------------------------------------------------

def config1(seed: int = 0) -> Problem:
    """fp32 RowMajor 128x64x256, A, B ~ U[0,1), C = 0, alpha = beta = 1."""
    return make_problem(128, 64, 256, dtype_ab=F32, dtype_cd=F32,
                        dist_a="uniform", dist_b="uniform", dist_c="zeros",
                        alpha=1.0, beta=1.0, seed=seed)


def config1_ones(n: int = 1024, dtype: str = F32) -> Problem:
    """All-ones n x n x n with C = 1, alpha = beta = 1 (closed form D = K + 1)."""
    return make_problem(n, n, n, dtype_ab=dtype, dtype_cd=dtype,
                        dist_a="ones", dist_b="ones", dist_c="ones",
                        alpha=1.0, beta=1.0)


def config2(seed: int = 0, n: int = 1024) -> Problem:
    """fp16 RowMajor n^3, A, B, C ~ N(0,1), alpha = beta = 1 (ReLU epilogue)."""
    return make_problem(n, n, n, dtype_ab=F16, dtype_cd=F16,
                        dist_c="normal", alpha=1.0, beta=1.0, seed=seed)


GROUPED_NK = (128, 256, 512, 1024, 4096)


def config3_shapes(seed: int = 0, count: int = 64) -> List[Tuple[int, int, int]]:
    """M uniform in {32, ..., 2048} step 32; N, K uniform in GROUPED_NK."""
    rng = np.random.default_rng(seed)
    Ms = rng.integers(1, 65, size=count) * 32
    Ns = rng.choice(GROUPED_NK, size=count)
    Ks = rng.choice(GROUPED_NK, size=count)
    return [(int(m), int(n), int(k)) for m, n, k in zip(Ms, Ns, Ks)]


def config3(seed: int = 0, count: int = 64,
            shapes: Optional[List[Tuple[int, int, int]]] = None) -> List[Problem]:
    """Grouped fp16 RowMajor problems, entries ~ N(0,1), beta = 0."""
    shapes = config3_shapes(seed, count) if shapes is None else shapes
    rng = np.random.default_rng(seed + 1)
    return [make_problem(m, n, k, dtype_ab=F16, dtype_cd=F16, rng=rng)
            for (m, n, k) in shapes]


# Transformer-layer bf16 GEMMs (hidden 8192, FFN 28672, 64 q / 8 kv heads of 128)
LAYER_SHAPES = {
    "qkv": (4096, 10240, 8192),
    "o": (4096, 8192, 8192),
    "gate_up": (4096, 57344, 8192),
    "down": (4096, 8192, 28672),
}


def config4(name: str, seed: int = 0, lb: str = COL, scale: int = 1) -> Problem:
    """bf16 A ~ N(0,1), weights ~ N(0, 0.02^2); B stored [N, K] (ColumnMajor)
    by default, like nn.Linear weights. ``scale`` divides M (for quick runs)."""
    M, N, K = LAYER_SHAPES[name]
    return make_problem(M // scale, N, K, dtype_ab=BF16, dtype_cd=BF16,
                        la=ROW, lb=lb, std_b=0.02, seed=seed)


DECODE_MS = (16, 64, 128)
DECODE_NK = ((8192, 28672), (57344, 8192))


def config5(M: int, N: int, K: int, seed: int = 0) -> Problem:
    """fp8 e4m3 A, B ~ N(0,1) quantized per tensor, bf16 D, beta = 0; B [N, K]."""
    return make_problem(M, N, K, dtype_ab=F8, dtype_cd=BF16, la=ROW, lb=COL,
                        seed=seed)


# ---------------------------------------------------------------------------
# MX (OCP Microscaling v1.0) inputs: e4m3 elements, one E8M0 scale per 32
# consecutive elements along K
# ---------------------------------------------------------------------------

MX_BLOCK = 32
E4M3_EMAX = 8          # largest e4m3 binade: 448 = 1.75 * 2^8
E2M1_EMAX = 2          # largest e2m1 binade: 6 = 1.5 * 2^2


def e2m1_codes(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even cast of values to OCP FP4 E2M1 codes (sign in
    bit 3; magnitudes beyond 6 saturate to 6): the storage cast of the MXFP4
    elements. A tie goes to the code with a zero fraction bit."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), E2M1_MAX)
    lo = np.clip(np.searchsorted(E2M1_GRID, a, side="right") - 1, 0, 7)
    hi = np.minimum(lo + 1, 7)
    d_lo = a - E2M1_GRID[lo]
    d_hi = E2M1_GRID[hi] - a
    up = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0) & (hi != lo))
    mag = np.where(up, hi, lo).astype(np.uint8)
    return mag | np.where(np.signbit(x) & (mag != 0), 8, 0).astype(np.uint8)


def pack_e2m1(codes: np.ndarray) -> torch.Tensor:
    """Storage [R, C] 4-bit codes -> [R, C/2] bytes, element 2t of a row in
    the low nibble of byte t (C even)."""
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    assert c.shape[-1] % 2 == 0
    return torch.from_numpy(np.ascontiguousarray((c[..., 0::2] & 15) | ((c[..., 1::2] & 15) << 4)))


def unpack_e2m1(packed: np.ndarray) -> np.ndarray:
    """Inverse of pack_e2m1: [R, C/2] bytes -> [R, C] 4-bit codes."""
    b = np.asarray(packed, dtype=np.uint8)
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = b & 15
    out[..., 1::2] = b >> 4
    return out


def mx_quantize(x32: np.ndarray, emax: int = E4M3_EMAX) -> Tuple[np.ndarray, torch.Tensor]:
    """Quantize logical [R, K] fp32 rows block by block (the MX conversion):
    shared exponent floor(log2(amax)) - emax per 32-element block (emax 8 for
    e4m3, 2 for e2m1), stored as the E8M0 code e + 127 (clamped to 0..254; an
    all-zero block gets 127); the elements x / 2^e are then cast to the
    element type (RNE, saturating) by the caller. Returns (elements as
    logical fp32 [R, K] before that cast, codes [R, K/32] uint8)."""
    R, K = x32.shape
    assert K % MX_BLOCK == 0
    blk = x32.reshape(R, K // MX_BLOCK, MX_BLOCK).astype(np.float64)
    amax = np.abs(blk).max(axis=2)
    safe = np.where(amax > 0, amax, 1.0)
    e = np.where(amax > 0, np.floor(np.log2(safe)) - emax, 0.0)
    code = np.clip(e + 127, 0, 254).astype(np.uint8)
    q = blk / np.exp2(code.astype(np.float64) - 127)[:, :, None]
    return q.reshape(R, K).astype(np.float32), torch.from_numpy(np.ascontiguousarray(code))


def mx_elements(q32: np.ndarray, layout: str, elem: str) -> torch.Tensor:
    """Logical MX elements (already divided by their block scales) ->
    storage in ``layout``: e4m3, or e2m1 codes packed two per byte along the
    storage's contiguous dimension (along K for A RowMajor / B ColumnMajor,
    the layouts the FP4 tile kernels take)."""
    if elem == F8:
        return cast(to_storage(q32, layout), F8)
    return pack_e2m1(e2m1_codes(to_storage(q32, layout)))


def make_mx_problem(M: int, N: int, K: int, *, la: str = ROW, lb: str = COL, lc: str = ROW,
                    dist_c: Optional[str] = None, alpha: float = 1.0, beta: float = 0.0,
                    dist_bias: Optional[str] = None, std_b: float = 1.0,
                    seed: int = 0, rng=None, elem: str = F8) -> Problem:
    """MXFP8 (elem f8e4m3) or MXFP4 (elem f4e2m1) problem: A, B ~ N(0,1) (B
    times std_b) quantized per 32-block of K; bf16 C / D. Draw order A, B, C,
    bias as in make_problem. MXFP4 elements are packed two per byte along
    each operand's contiguous dimension (see mx_elements)."""
    rng = np.random.default_rng(seed) if rng is None else rng
    a32 = _draw(rng, (M, K), "normal")
    b32 = _draw(rng, (K, N), "normal", std_b)
    c = None
    if dist_c is not None:
        c = cast(to_storage(_draw(rng, (M, N), dist_c), lc), BF16)
    bias = cast(_draw(rng, (N,), dist_bias), BF16) if dist_bias is not None else None
    emax = E4M3_EMAX if elem == F8 else E2M1_EMAX
    qa, xa = mx_quantize(a32, emax)
    qbt, xb = mx_quantize(np.ascontiguousarray(b32.T), emax)
    A = mx_elements(qa, la, elem)
    B = mx_elements(np.ascontiguousarray(qbt.T), lb, elem)
    return Problem(M, N, K, A, B, c, alpha, beta, None, None, elem, BF16, la, lb, lc, bias,
                   xa, xb)


def mx_integer_problem(M: int, N: int, K: int, *, la: str = ROW, lb: str = COL,
                       lc: str = ROW, lo: int = -2, hi: int = 2, emin: int = -2,
                       emax: int = 2, with_c: bool = True, beta: float = 1.0,
                       with_bias: bool = False, seed: int = 0, elem: str = F8) -> Problem:
    """MX problem with integer elements in [lo, hi] and scale codes
    127 + U{emin..emax}: every scaled product and partial sum is a small
    dyadic number, exact in fp32. For MXFP4 (elem f4e2m1) every integer in
    [-4, 4] is an e2m1 value."""
    rng = np.random.default_rng(seed)
    a32 = rng.integers(lo, hi + 1, size=(M, K)).astype(np.float32)
    b32 = rng.integers(lo, hi + 1, size=(K, N)).astype(np.float32)
    c = None
    if with_c:
        c = cast(to_storage(rng.integers(lo, hi + 1, size=(M, N)).astype(np.float32), lc), BF16)
    bias = None
    if with_bias:
        bias = cast(rng.integers(lo, hi + 1, size=(N,)).astype(np.float32), BF16)
    nb = K // MX_BLOCK
    xa = torch.from_numpy((127 + rng.integers(emin, emax + 1, size=(M, nb))).astype(np.uint8))
    xb = torch.from_numpy((127 + rng.integers(emin, emax + 1, size=(N, nb))).astype(np.uint8))
    if elem == F4:
        assert -4 <= lo <= hi <= 4
    A = mx_elements(a32, la, elem)
    B = mx_elements(b32, lb, elem)
    return Problem(M, N, K, A, B, c, 1.0, beta if with_c else 0.0, None, None, elem, BF16,
                   la, lb, lc, bias, xa, xb)


def config4_device(name: str, device, seed: int = 0, lb: str = COL):
    """config4 drawn with torch on ``device`` (full-size benchmark inputs; the
    same distributions, another generator): A ~ N(0,1) [M, K] bf16, W ~
    N(0, 0.02^2) stored [N, K] (lb ColumnMajor) or [K, N] (lb RowMajor).
    Returns (M, N, K, A, B)."""
    M, N, K = LAYER_SHAPES[name]
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    A = torch.randn((M, K), generator=gen, device=device, dtype=torch.float32).to(torch.bfloat16)
    w = torch.randn((N, K), generator=gen, device=device, dtype=torch.float32).mul_(0.02)
    B = (w if lb == COL else w.t()).to(torch.bfloat16).contiguous()
    del w
    return M, N, K, A, B


def config5_device(M: int, N: int, K: int, device, seed: int = 0):
    """config5 drawn with torch on ``device``: A [M, K] and B stored [N, K],
    N(0,1) entries, each quantized to e4m3 with the per-tensor scale rule of
    quantize_e4m3 (s = amax / 448). Returns (A, B, s_a, s_b)."""
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    out = []
    for shape in ((M, K), (N, K)):
        x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
        amax = float(x.abs().max())
        s = amax / E4M3_MAX if amax > 0 else 1.0
        out.append((x.div_(s).to(torch.float8_e4m3fn), float(np.float32(s))))
        del x
    (A, sa), (B, sb) = out
    return A, B, sa, sb


def mx_quantize_device(x: torch.Tensor) -> Tuple[torch.Tensor, torch.Tensor]:
    """The MX conversion of mx_quantize done with torch ops on x's device
    (for full-size benchmark inputs): logical [R, K] rows -> (e4m3 elements
    [R, K], E8M0 codes [R, K/32] uint8); same shared-exponent rule, RNE
    saturating element cast."""
    R, K = x.shape
    assert K % MX_BLOCK == 0
    blk = x.float().reshape(R, K // MX_BLOCK, MX_BLOCK)
    amax = blk.abs().amax(dim=2)
    e = torch.where(amax > 0, torch.floor(torch.log2(torch.where(amax > 0, amax,
                                                                  torch.ones_like(amax))))
                    - E4M3_EMAX, torch.zeros_like(amax))
    code = (e + 127).clamp(0, 254)
    q = (blk / torch.exp2(code - 127).unsqueeze(2)).clamp(-E4M3_MAX, E4M3_MAX)
    return (q.reshape(R, K).to(torch.float8_e4m3fn),
            code.to(torch.uint8).contiguous())


def mx_layer_device(name: str, device, seed: int = 0):
    """MXFP8 version of a transformer-layer GEMM, drawn on ``device``:
    A ~ N(0,1) [M, K] RowMajor, W ~ N(0, 0.02^2) stored [N, K] (ColumnMajor
    B), both MX-quantized along K. Returns (M, N, K, A, B, scales_a, scales_b)."""
    M, N, K = LAYER_SHAPES[name]
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    a = torch.randn((M, K), generator=gen, device=device, dtype=torch.float32)
    A, xa = mx_quantize_device(a)
    del a
    w = torch.randn((N, K), generator=gen, device=device, dtype=torch.float32) * 0.02
    B, xb = mx_quantize_device(w)
    return M, N, K, A, B, xa, xb


def mx4_quantize_device(x: torch.Tensor) -> Tuple[torch.Tensor, torch.Tensor]:
    """The MXFP4 conversion of mx_quantize / e2m1_codes / pack_e2m1 done with
    torch ops on x's device (full-size benchmark inputs): logical [R, K] rows
    -> (e2m1 codes packed two per byte along K [R, K/2] uint8, E8M0 codes
    [R, K/32] uint8); same shared-exponent rule (emax 2), RNE saturating
    element cast with ties to the even code."""
    R, K = x.shape
    assert K % MX_BLOCK == 0
    blk = x.float().reshape(R, K // MX_BLOCK, MX_BLOCK)
    amax = blk.abs().amax(dim=2)
    e = torch.where(amax > 0, torch.floor(torch.log2(torch.where(amax > 0, amax,
                                                                  torch.ones_like(amax))))
                    - E2M1_EMAX, torch.zeros_like(amax))
    code = (e + 127).clamp(0, 254)
    q = (blk / torch.exp2(code - 127).unsqueeze(2)).reshape(R, K)
    del blk
    grid = torch.tensor(E2M1_GRID, dtype=torch.float32, device=x.device)
    a = q.abs().clamp(max=E2M1_MAX)
    lo = (torch.bucketize(a, grid, right=True) - 1).clamp(0, 7)
    hi = (lo + 1).clamp(max=7)
    d_lo = a - grid[lo]
    d_hi = grid[hi] - a
    up = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0) & (hi != lo))
    mag = torch.where(up, hi, lo).to(torch.uint8)
    del a, d_lo, d_hi, up, lo, hi
    c = mag | torch.where(torch.signbit(q) & (mag != 0), 8, 0).to(torch.uint8)
    del q, mag
    packed = (c[:, 0::2] & 15) | ((c[:, 1::2] & 15) << 4)
    return packed.contiguous(), code.to(torch.uint8).contiguous()


def mx4_layer_device(name: str, device, seed: int = 0):
    """MXFP4 version of a transformer-layer GEMM, drawn on ``device`` like
    mx_layer_device and MXFP4-quantized along K. Returns (M, N, K, A, B,
    scales_a, scales_b) with A [M, K/2] and B [N, K/2] packed bytes."""
    M, N, K = LAYER_SHAPES[name]
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    a = torch.randn((M, K), generator=gen, device=device, dtype=torch.float32)
    A, xa = mx4_quantize_device(a)
    del a
    w = torch.randn((N, K), generator=gen, device=device, dtype=torch.float32) * 0.02
    B, xb = mx4_quantize_device(w)
    return M, N, K, A, B, xa, xb


# ---------------------------------------------------------------------------
# auxiliary tensor of the epilogue


def add_aux(p: Problem, op: str = "add", pos: str = "before", dist: str = "normal",
            seed: int = 0, lo: int = -3, hi: int = 3) -> Problem:
    """Attach an M x N auxiliary tensor (dtype_cd, layout p.lc) drawn from its
    own generator ``seed``, so the problem's other draws do not change.
    dist: "normal" N(0,1); "away" sign * U[0.5, 2) (bounded away from zero,
    for division); "int" integers in [lo, hi]; "int_nz" the same without 0;
    "ones"."""
    rng = np.random.default_rng(seed)
    shape = (p.M, p.N)
    if dist == "away":
        x = (rng.random(shape, dtype=np.float32) * np.float32(1.5) + np.float32(0.5))
        x = np.where(rng.random(shape) < 0.5, -x, x).astype(np.float32)
    elif dist in ("int", "int_nz"):
        x = rng.integers(lo, hi + 1, size=shape).astype(np.float32)
        if dist == "int_nz":
            x = np.where(x == 0, np.float32(hi), x).astype(np.float32)
    else:
        x = _draw(rng, shape, dist)
    p.aux = cast(to_storage(x, p.lc), p.dtype_cd)
    p.aux_op, p.aux_pos = op, pos
    return p
