"""CPU oracle for the GEMM D = alpha*A*B + beta*C -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline
leg may import this package. The GPU library never calls it and shares no
code with it; the product path fails loudly when its HIP library is missing.

The arithmetic lives in ``oracle.c`` (plain fp64 loops, its own format
decoders and its own round-to-nearest-even encoder); this module only
marshals numpy arrays through ctypes. Grouped GEMM is, by its definition on
the pages ("Python packages associated with CUTLASS", Current functionality:
grouped GEMM runs independent problems in one call), a loop of single GEMMs.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import List, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

DT = {"f32": 0, "f16": 1, "bf16": 2, "f8e4m3": 3, "e8m0": 4, "f4e2m1": 5}
LAYOUT = {"row": 0, "col": 1}

_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc into liboracle.so next to it."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC",
                               "-Wall", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        L = ctypes.CDLL(_LIB)
        i64p = ctypes.POINTER(ctypes.c_int64)
        vp = ctypes.c_void_p
        L.oracle_decode.restype = ctypes.c_double
        L.oracle_decode.argtypes = [ctypes.c_int, ctypes.c_uint32]
        L.oracle_encode.restype = ctypes.c_uint32
        L.oracle_encode.argtypes = [ctypes.c_int, ctypes.c_double]
        L.oracle_decode_n.argtypes = [ctypes.c_int, vp, ctypes.c_int64, vp]
        L.oracle_encode_n.argtypes = [ctypes.c_int, vp, ctypes.c_int64, vp]
        common = [ctypes.c_int] * 8 + [ctypes.c_int64] * 3 + [vp] * 7 + \
                 [ctypes.c_int] * 2 + [ctypes.c_float] * 4
        L.oracle_gemm_rows.restype = ctypes.c_int
        L.oracle_gemm_rows.argtypes = common + [i64p, ctypes.c_int64] + [vp] * 6
        L.oracle_gemm_entries.restype = ctypes.c_int
        L.oracle_gemm_entries.argtypes = common + [i64p, i64p, ctypes.c_int64] + [vp] * 6
        _lib = L
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def decode(dtype: str, bits) -> np.ndarray:
    """Exact fp64 values of storage bit patterns of ``dtype``."""
    b = np.ascontiguousarray(np.asarray(bits).astype(np.uint32))
    out = np.empty(b.shape, dtype=np.float64)
    lib().oracle_decode_n(DT[dtype], _ptr(b), b.size, _ptr(out))
    return out


def encode(dtype: str, values) -> np.ndarray:
    """Round-to-nearest-even bit patterns of fp64 ``values`` in ``dtype``."""
    v = np.ascontiguousarray(np.asarray(values, dtype=np.float64))
    out = np.empty(v.shape, dtype=np.uint32)
    lib().oracle_encode_n(DT[dtype], _ptr(v), v.size, _ptr(out))
    return out


class Result:
    """Oracle outputs for selected rows or entries."""

    def __init__(self, ref, S, d_bits, dtype_d, z_ref=None, z_S=None, z_bits=None):
        self.ref = ref          # fp64 unrounded epilogue value
        self.S = S              # |alpha s_A s_B| * sum_k |a b| (times the aux op's factor)
        self.d_bits = d_bits    # element_D bits of the once-rounded value
        self.dtype_d = dtype_d
        self.z_ref = z_ref      # the activation's input (the auxiliary store), fp64
        self.z_S = z_S          # its tolerance scale
        self.z_bits = z_bits    # its element_D bits

    @property
    def d_exact(self) -> np.ndarray:
        return decode(self.dtype_d, self.d_bits)

    @property
    def z_exact(self) -> np.ndarray:
        return decode(self.dtype_d, self.z_bits)


def _scalars(p):
    sa = 1.0 if p.scale_a is None else p.scale_a
    sb = 1.0 if p.scale_b is None else p.scale_b
    return float(p.alpha), float(p.beta), float(sa), float(sb)


# Activations of the epilogue (the codes the C oracle takes).
ACT = {"identity": 0, "relu": 1, "sigmoid": 2, "tanh": 3}
# The auxiliary tensor's elementwise op and its side of the activation.
AUX_OP = {"add": 0, "sub": 1, "mul": 2, "div": 3}
AUX_POS = {"before": 0, "after": 1}


def _operands(p):
    from synthetic import raw   # storage bytes only
    A = raw(p.A)
    B = raw(p.B)
    C = raw(p.C) if (p.C is not None and p.beta != 0.0) else None
    bias = raw(p.bias) if getattr(p, "bias", None) is not None else None
    xa = raw(p.mx_a) if getattr(p, "mx_a", None) is not None else None
    xb = raw(p.mx_b) if getattr(p, "mx_b", None) is not None else None
    aux = raw(p.aux) if getattr(p, "aux", None) is not None else None
    return A, B, C, bias, xa, xb, aux


def _aux_args(p, aux):
    op = AUX_OP[getattr(p, "aux_op", "add")]
    pos = AUX_POS[getattr(p, "aux_pos", "before")]
    return _ptr(aux), op, pos


def _outputs(shape):
    return (np.empty(shape, dtype=np.float64), np.empty(shape, dtype=np.float64),
            np.empty(shape, dtype=np.uint32), np.empty(shape, dtype=np.float64),
            np.empty(shape, dtype=np.float64), np.empty(shape, dtype=np.uint32))


def _act_code(relu: bool, act: Optional[str]) -> int:
    if act is None:
        return ACT["relu"] if relu else ACT["identity"]
    if relu and act != "relu":
        raise ValueError("relu=True conflicts with act=%r" % act)
    return ACT[act]


def _head(p, relu, act=None):
    return (DT[p.dtype_ab], DT[p.dtype_ab], DT[p.dtype_cd], DT[p.dtype_cd],
            LAYOUT[p.la], LAYOUT[p.lb], LAYOUT[p.lc], _act_code(relu, act),
            p.M, p.N, p.K)


def gemm(p, relu: bool = False, rows: Optional[Sequence[int]] = None,
         act: Optional[str] = None) -> Result:
    """Full rows of D for the problem ``p`` (a ``synthetic.Problem``; its
    ``bias``, if any, is added to every row before the activation; its
    ``mx_a`` / ``mx_b``, if set, are the E8M0 block scales of an MX problem;
    its ``aux``, if set, is the M x N auxiliary tensor combined by
    ``aux_op`` on the ``aux_pos`` side of the activation, and the result
    also carries the auxiliary store Z).

    ``rows`` = None computes all M rows; outputs are [n_rows, N] arrays.
    ``act`` names the activation ("identity", "relu", "sigmoid", "tanh");
    ``relu=True`` is shorthand for act="relu".
    """
    A, B, C, bias, xa, xb, aux = _operands(p)
    al, be, sa, sb = _scalars(p)
    if rows is None:
        rows_arr, n = None, p.M
    else:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        n = rows_arr.size
    outs = _outputs((n, p.N))
    rp = None if rows_arr is None else rows_arr.ctypes.data_as(
        ctypes.POINTER(ctypes.c_int64))
    rc = lib().oracle_gemm_rows(*_head(p, relu, act), _ptr(A), _ptr(B), _ptr(C),
                                _ptr(bias), _ptr(xa), _ptr(xb), *_aux_args(p, aux),
                                al, be, sa, sb, rp, n, *(_ptr(o) for o in outs))
    if rc != 0:
        raise ValueError("oracle_gemm_rows: bad arguments")
    ref, S, d, zr, zs, zb = outs
    return Result(ref, S, d, p.dtype_cd, zr, zs, zb)


def gemm_entries(p, ii, jj, relu: bool = False, act: Optional[str] = None) -> Result:
    """Selected outputs D[ii[t], jj[t]], each computed on its own."""
    A, B, C, bias, xa, xb, aux = _operands(p)
    al, be, sa, sb = _scalars(p)
    ii = np.ascontiguousarray(np.asarray(ii, dtype=np.int64))
    jj = np.ascontiguousarray(np.asarray(jj, dtype=np.int64))
    n = ii.size
    outs = _outputs(n)
    P = ctypes.POINTER(ctypes.c_int64)
    rc = lib().oracle_gemm_entries(*_head(p, relu, act), _ptr(A), _ptr(B), _ptr(C),
                                   _ptr(bias), _ptr(xa), _ptr(xb), *_aux_args(p, aux),
                                   al, be, sa, sb, ii.ctypes.data_as(P),
                                   jj.ctypes.data_as(P), n, *(_ptr(o) for o in outs))
    if rc != 0:
        raise ValueError("oracle_gemm_entries: bad arguments")
    ref, S, d, zr, zs, zb = outs
    return Result(ref, S, d, p.dtype_cd, zr, zs, zb)


def grouped(problems: List, relu: bool = False, act: Optional[str] = None) -> List[Result]:
    """Grouped GEMM = the independent single GEMMs, one after another."""
    return [gemm(p, relu, act=act) for p in problems]


def batched(problems: List, relu: bool = False, act: Optional[str] = None) -> List[Result]:
    """Batched GEMM ("CUTLASS Python接口", batched GEMM: a batch count and a
    stride per operand) = one independent GEMM per batch index, all of one
    shape; how the batch is laid out in memory (the strides) is the caller's
    packing, not arithmetic, so each entry is passed as its own problem."""
    if problems and any((p.M, p.N, p.K) != (problems[0].M, problems[0].N, problems[0].K)
                        for p in problems):
        raise ValueError("batched GEMM problems share one M x N x K")
    return [gemm(p, relu, act=act) for p in problems]
