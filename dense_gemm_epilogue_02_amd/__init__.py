"""Python binding of the gfx950 GEMM library (``libmi355_gemm.so``).

Argument marshalling only: every step of D = epi(alpha*A*B + beta*C) runs in
the library's HIP kernels. The functions keep the C ABI's names
(``gemm_plan_create``, ``gemm_plan_run``, ``gemm_plan_run_scaled``,
``grouped_gemm_run``, ...); ``Plan`` and ``gemm``/``grouped_gemm`` are small
conveniences that take torch tensors, check their sizes against M, N, K on the
host (so no kernel is launched on a buffer that is too small), and pass their
device pointers and torch's current HIP stream.

There is no fallback: if the shared library is missing, importing this module
raises with the command that builds it.
"""
from __future__ import annotations

import ctypes
import os
from enum import IntEnum
from typing import Iterable, List, Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmi355_gemm.so")


class Dtype(IntEnum):
    F32 = 0
    F16 = 1
    BF16 = 2
    F8_E4M3 = 3
    F4_E2M1 = 4   # packed two per byte (uint8 tensors), MX runs only


class Layout(IntEnum):
    ROW_MAJOR = 0
    COL_MAJOR = 1


class Epilogue(IntEnum):
    LINEAR = 0
    RELU = 1
    SIGMOID = 2
    TANH = 3


class Status(IntEnum):
    OK = 0
    INVALID_ARG = 1
    UNSUPPORTED = 2
    HIP_ERROR = 3
    OUT_OF_MEMORY = 4
    NOT_INITIALIZED = 5


class Schedule(IntEnum):
    AUTO = 0
    DATA_PARALLEL = 1
    STREAM_K = 2
    HYBRID = 3
    SPLIT_K = 4


class Tile(IntEnum):
    AUTO = 0
    T256x256 = 1
    T128x128 = 2
    T64x256 = 3
    T32x256 = 4
    GENERIC = 5
    WHOLEK = 6


class GemmError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{Status(status).name}: {message}")
        self.status = Status(status)


class gemm_problem(ctypes.Structure):
    _fields_ = [("M", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64),
                ("A", ctypes.c_void_p), ("B", ctypes.c_void_p), ("C", ctypes.c_void_p),
                ("D", ctypes.c_void_p)]


class gemm_config(ctypes.Structure):
    _fields_ = [("schedule", ctypes.c_int), ("tile", ctypes.c_int), ("sk_grid", ctypes.c_int32),
                ("grid", ctypes.c_int32), ("us", ctypes.c_float)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'` "
            "or `python dense_gemm_epilogue_02_amd/build.py` (needs hipcc for gfx950)")
    # One HIP runtime per process: torch ships its own libamdhip64 and asks for
    # it by its unversioned file name, so if this library were loaded first its
    # libamdhip64.so.7 from ROCm would stay beside torch's as a second runtime
    # with its own device state. Loading torch first makes the soname resolve to
    # the copy torch already holds.
    import torch  # noqa: F401
    L = ctypes.CDLL(LIB_PATH)
    i32, i64, f32, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p
    st = ctypes.c_int
    L.gemm_plan_create.restype = st
    L.gemm_plan_create.argtypes = [ctypes.POINTER(vp)] + [ctypes.c_int] * 9
    L.gemm_plan_create_simple.restype = st
    L.gemm_plan_create_simple.argtypes = [ctypes.POINTER(vp)] + [ctypes.c_int] * 3
    L.gemm_plan_destroy.restype = st
    L.gemm_plan_destroy.argtypes = [vp]
    L.gemm_plan_set_config.restype = st
    L.gemm_plan_set_config.argtypes = [vp, ctypes.c_int, ctypes.c_int, i32]
    L.gemm_plan_run.restype = st
    L.gemm_plan_run.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, f32, f32, vp]
    L.gemm_plan_run_noalloc.restype = st
    L.gemm_plan_run_noalloc.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, f32, f32, vp]
    L.gemm_plan_run_scaled.restype = st
    L.gemm_plan_run_scaled.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, f32, f32, vp, vp, vp]
    L.gemm_plan_run_ex.restype = st
    L.gemm_plan_run_ex.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, f32, f32, vp, vp, vp]
    L.gemm_plan_run_mx.restype = st
    L.gemm_plan_run_mx.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, f32, f32, vp, vp, vp]
    L.gemm_plan_run_aux.restype = st
    L.gemm_plan_run_aux.argtypes = [vp, vp, vp, vp, vp, vp, vp, ctypes.c_int, ctypes.c_int, vp,
                                    i64, i64, i64, f32, f32, vp, vp, vp]
    L.gemm_plan_run_batched.restype = st
    L.gemm_plan_run_batched.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64,
                                        i64, i64, f32, f32, vp, vp, vp]
    L.grouped_gemm_run.restype = st
    L.grouped_gemm_run.argtypes = [vp, ctypes.POINTER(gemm_problem), i32, f32, f32, vp]
    L.gemm_plan_profile.restype = st
    L.gemm_plan_profile.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, f32, f32, i32,
                                    ctypes.POINTER(gemm_config), i32, ctypes.POINTER(i32), vp]
    L.gemm_plan_cache_export.restype = st
    L.gemm_plan_cache_export.argtypes = [vp, ctypes.c_char_p, i32, ctypes.POINTER(i32)]
    L.gemm_plan_cache_import.restype = st
    L.gemm_plan_cache_import.argtypes = [vp, ctypes.c_char_p]
    L.gemm_plan_cache_size.restype = i32
    L.gemm_plan_cache_size.argtypes = [vp]
    L.gemm_plan_cache_clear.restype = st
    L.gemm_plan_cache_clear.argtypes = [vp]
    L.gemm_plan_describe.restype = st
    L.gemm_plan_describe.argtypes = [vp, i64, i64, i64, i32, ctypes.c_char_p, i32]
    L.gemm_plan_describe_batched.restype = st
    L.gemm_plan_describe_batched.argtypes = [vp, i64, i64, i64, i64, i32, ctypes.c_char_p, i32]
    L.gemm_last_error.restype = ctypes.c_char_p
    L.gemm_last_error.argtypes = []
    L.gemm_status_string.restype = ctypes.c_char_p
    L.gemm_status_string.argtypes = [ctypes.c_int]
    L.gemm_supported_count.restype = i32
    L.gemm_supported_count.argtypes = []
    L.gemm_supported_get.restype = st
    L.gemm_supported_get.argtypes = [i32] + [ctypes.POINTER(ctypes.c_int)] * 5
    L.gemm_version.restype = ctypes.c_char_p
    L.gemm_version.argtypes = []
    return L


lib = _load()

EXPORTED = ("gemm_plan_create", "gemm_plan_create_simple", "gemm_plan_destroy",
            "gemm_plan_set_config", "gemm_plan_run", "gemm_plan_run_noalloc", "gemm_plan_run_scaled",
            "gemm_plan_run_ex", "gemm_plan_run_mx", "gemm_plan_run_aux",
            "gemm_plan_run_batched", "grouped_gemm_run", "gemm_plan_profile",
            "gemm_plan_cache_export", "gemm_plan_cache_import", "gemm_plan_cache_size",
            "gemm_plan_cache_clear", "gemm_plan_describe", "gemm_plan_describe_batched",
            "gemm_last_error",
            "gemm_status_string", "gemm_supported_count", "gemm_supported_get",
            "gemm_version")


def _check(status: int):
    if status != 0:
        raise GemmError(status, lib.gemm_last_error().decode())


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# ---- same-name wrappers of the C ABI ----------------------------------------

def gemm_plan_create(element_a, element_b, element_c, element_d, element_acc,
                     layout_a, layout_b, layout_c, epilogue) -> int:
    h = ctypes.c_void_p()
    _check(lib.gemm_plan_create(ctypes.byref(h), int(element_a), int(element_b),
                                int(element_c), int(element_d), int(element_acc),
                                int(layout_a), int(layout_b), int(layout_c), int(epilogue)))
    return h.value


def gemm_plan_create_simple(element, layout, epilogue) -> int:
    h = ctypes.c_void_p()
    _check(lib.gemm_plan_create_simple(ctypes.byref(h), int(element), int(layout), int(epilogue)))
    return h.value


def gemm_plan_destroy(plan: int) -> None:
    _check(lib.gemm_plan_destroy(plan))


def gemm_plan_set_config(plan: int, schedule=Schedule.AUTO, tile=Tile.AUTO, sk_grid: int = 0):
    _check(lib.gemm_plan_set_config(plan, int(schedule), int(tile), int(sk_grid)))


def gemm_plan_run(plan: int, A, B, C, D, M: int, N: int, K: int, alpha: float = 1.0,
                  beta: float = 0.0, stream=None) -> None:
    _check(lib.gemm_plan_run(plan, _ptr(A), _ptr(B), _ptr(C), _ptr(D), M, N, K, alpha, beta,
                             _stream(stream)))


def gemm_plan_run_noalloc(plan: int, A, B, C, D, M: int, N: int, K: int, alpha: float = 1.0,
                          beta: float = 0.0, stream=None) -> None:
    _check(lib.gemm_plan_run_noalloc(plan, _ptr(A), _ptr(B), _ptr(C), _ptr(D), M, N, K, alpha,
                                     beta, _stream(stream)))


def gemm_plan_run_scaled(plan: int, A, B, C, D, M: int, N: int, K: int, alpha: float,
                         beta: float, scale_a, scale_b, stream=None) -> None:
    _check(lib.gemm_plan_run_scaled(plan, _ptr(A), _ptr(B), _ptr(C), _ptr(D), M, N, K, alpha,
                                    beta, _ptr(scale_a), _ptr(scale_b), _stream(stream)))


def gemm_plan_run_ex(plan: int, A, B, C, D, bias, M: int, N: int, K: int, alpha: float,
                     beta: float, scale_a=None, scale_b=None, stream=None) -> None:
    _check(lib.gemm_plan_run_ex(plan, _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(bias), M, N, K,
                                alpha, beta, _ptr(scale_a), _ptr(scale_b), _stream(stream)))


def gemm_plan_run_mx(plan: int, A, B, C, D, bias, M: int, N: int, K: int, alpha: float,
                     beta: float, mx_scale_a, mx_scale_b, stream=None) -> None:
    _check(lib.gemm_plan_run_mx(plan, _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(bias), M, N, K,
                                alpha, beta, _ptr(mx_scale_a), _ptr(mx_scale_b),
                                _stream(stream)))


# gemm_aux_op / gemm_aux_pos
AUX_OP = {"add": 0, "sub": 1, "mul": 2, "div": 3}
AUX_POS = {"before": 0, "after": 1}


def gemm_plan_run_aux(plan: int, A, B, C, D, bias, aux, aux_op: int, aux_pos: int, aux_out,
                      M: int, N: int, K: int, alpha: float, beta: float, scale_a=None,
                      scale_b=None, stream=None) -> None:
    _check(lib.gemm_plan_run_aux(plan, _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(bias), _ptr(aux),
                                 int(aux_op), int(aux_pos), _ptr(aux_out), M, N, K, alpha, beta,
                                 _ptr(scale_a), _ptr(scale_b), _stream(stream)))


def gemm_plan_run_batched(plan: int, A, B, C, D, bias, M: int, N: int, K: int, batch: int,
                          stride_a: int, stride_b: int, stride_c: int, stride_d: int,
                          alpha: float, beta: float, scale_a=None, scale_b=None,
                          stream=None) -> None:
    _check(lib.gemm_plan_run_batched(plan, _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(bias), M, N,
                                     K, batch, stride_a, stride_b, stride_c, stride_d, alpha,
                                     beta, _ptr(scale_a), _ptr(scale_b), _stream(stream)))


def grouped_gemm_run(plan: int, problems: Sequence[tuple], alpha: float = 1.0,
                     beta: float = 0.0, stream=None) -> None:
    """problems: sequence of (M, N, K, A, B, C, D) with tensors or raw pointers."""
    arr = (gemm_problem * max(1, len(problems)))()
    for i, (M, N, K, A, B, C, D) in enumerate(problems):
        arr[i] = gemm_problem(M, N, K, _ptr(A), _ptr(B), _ptr(C), _ptr(D))
    _check(lib.grouped_gemm_run(plan, arr, len(problems), alpha, beta, _stream(stream)))


def gemm_plan_profile(plan: int, A, B, C, D, M: int, N: int, K: int, alpha: float = 1.0,
                      beta: float = 0.0, iters: int = 10, max_results: int = 32,
                      stream=None) -> list:
    """Time every distinct launch of the plan for M x N x K; fastest first.
    The fastest is cached in the plan for later runs of this shape."""
    arr = (gemm_config * max(1, max_results))()
    n = ctypes.c_int32(0)
    _check(lib.gemm_plan_profile(plan, _ptr(A), _ptr(B), _ptr(C), _ptr(D), M, N, K, alpha, beta,
                                 iters, arr, max_results, ctypes.byref(n), _stream(stream)))
    return [dict(schedule=Schedule(c.schedule), tile=Tile(c.tile), sk_grid=c.sk_grid,
                 grid=c.grid, us=c.us) for c in arr[:min(n.value, max_results)]]


def gemm_plan_cache_export(plan: int) -> str:
    need = ctypes.c_int32(0)
    _check(lib.gemm_plan_cache_export(plan, None, 0, ctypes.byref(need)))
    buf = ctypes.create_string_buffer(need.value)
    _check(lib.gemm_plan_cache_export(plan, buf, len(buf), ctypes.byref(need)))
    return buf.value.decode()


def gemm_plan_cache_import(plan: int, text: str) -> None:
    _check(lib.gemm_plan_cache_import(plan, text.encode()))


def gemm_plan_cache_size(plan: int) -> int:
    return lib.gemm_plan_cache_size(plan)


def gemm_plan_cache_clear(plan: int) -> None:
    _check(lib.gemm_plan_cache_clear(plan))


def gemm_plan_describe(plan: int, M: int, N: int, K: int, num_cus: int = 0) -> dict:
    import json
    buf = ctypes.create_string_buffer(512)
    _check(lib.gemm_plan_describe(plan, M, N, K, num_cus, buf, len(buf)))
    return json.loads(buf.value.decode())


def gemm_plan_describe_batched(plan: int, M: int, N: int, K: int, batch: int,
                               num_cus: int = 0) -> dict:
    import json
    buf = ctypes.create_string_buffer(512)
    _check(lib.gemm_plan_describe_batched(plan, M, N, K, batch, num_cus, buf, len(buf)))
    return json.loads(buf.value.decode())


def gemm_last_error() -> str:
    return lib.gemm_last_error().decode()


def gemm_status_string(status: int) -> str:
    return lib.gemm_status_string(int(status)).decode()


def gemm_supported_count() -> int:
    return lib.gemm_supported_count()


def gemm_supported_get(i: int):
    v = [ctypes.c_int() for _ in range(5)]
    _check(lib.gemm_supported_get(i, *[ctypes.byref(x) for x in v]))
    return tuple(Dtype(x.value) for x in v)


def gemm_version() -> str:
    return lib.gemm_version().decode()


# ---- tensor conveniences ------------------------------------------------------

_TORCH_DT = {"f32": Dtype.F32, "f16": Dtype.F16, "bf16": Dtype.BF16, "f8e4m3": Dtype.F8_E4M3,
             "f4e2m1": Dtype.F4_E2M1}
_LAYOUT = {"row": Layout.ROW_MAJOR, "col": Layout.COL_MAJOR}


def _dtype_of(t) -> Dtype:
    import torch
    m = {torch.float32: Dtype.F32, torch.float16: Dtype.F16, torch.bfloat16: Dtype.BF16,
         torch.float8_e4m3fn: Dtype.F8_E4M3, torch.uint8: Dtype.F4_E2M1}
    if t.dtype not in m:
        raise TypeError(f"unsupported tensor dtype {t.dtype}")
    return m[t.dtype]


def _need(t, n: int, name: str, dtype: Dtype):
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (packed storage)")
    if _dtype_of(t) != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, plan expects {dtype.name}")
    per = 2 if dtype == Dtype.F4_E2M1 else 1   # FP4: two elements per byte
    if t.numel() * per < n:
        raise ValueError(f"{name} holds {t.numel() * per} elements, needs {n}")


class GroupedProblems:
    """A grouped problem list checked against a plan once and packed into the
    C array of gemm_problem (the tensors are kept alive with it), so repeated
    launches of the same list cost no per-problem Python work."""

    def __init__(self, plan: "Plan", problems: Iterable[tuple], beta: float = 0.0):
        probs = list(problems)
        for (M, N, K, A, B, C, D) in probs:
            plan.check(A, B, C, D, M, N, K, beta)
        self.plan = plan
        self.beta = beta
        self.count = len(probs)
        self.arr = (gemm_problem * max(1, len(probs)))()
        for i, (M, N, K, A, B, C, D) in enumerate(probs):
            self.arr[i] = gemm_problem(M, N, K, _ptr(A), _ptr(B), _ptr(C), _ptr(D))
        self._keep = probs


class PreparedRun:
    """One gemm_plan_run call checked against its plan once, its C arguments
    converted once (the tensors are kept alive with it, the stream is the one
    given or current when prepared): calling it launches the GEMM again on
    the same buffers with no per-call Python checks. For small, launch-bound
    problems run many times, as a serving loop holds its buffers; the
    buffers' contents may change between calls, their shapes and addresses
    may not."""

    def __init__(self, plan: "Plan", A, B, C, D, M: int, N: int, K: int, alpha: float = 1.0,
                 beta: float = 0.0, stream=None):
        plan.check(A, B, C, D, M, N, K, beta)
        self.plan = plan
        vals = (plan.handle, _ptr(A), _ptr(B), _ptr(C), _ptr(D), M, N, K, alpha, beta,
                _stream(stream))
        self._args = tuple(t(v) for t, v in zip(lib.gemm_plan_run.argtypes, vals))
        self._keep = (A, B, C, D)

    def __call__(self) -> None:
        if self.plan.handle is None:   # the packed handle would be a dangling one
            raise GemmError(Status.NOT_INITIALIZED, "PreparedRun: its plan was closed")
        _check(lib.gemm_plan_run(*self._args))


class Plan:
    """A plan bound to element types, layouts and epilogue (reusable across shapes)."""

    _ACT = {"linear": Epilogue.LINEAR, "identity": Epilogue.LINEAR, "relu": Epilogue.RELU,
            "sigmoid": Epilogue.SIGMOID, "tanh": Epilogue.TANH}

    def __init__(self, dtype_ab="bf16", dtype_cd=None, la="row", lb="row", lc="row",
                 relu: bool = False, activation: Optional[str] = None):
        dtype_cd = dtype_cd or ("bf16" if dtype_ab in ("f8e4m3", "f4e2m1") else dtype_ab)
        self.dab, self.dcd = _TORCH_DT[dtype_ab], _TORCH_DT[dtype_cd]
        if activation is None:
            epi = Epilogue.RELU if relu else Epilogue.LINEAR
        else:
            if relu and activation != "relu":
                raise ValueError(f"relu=True conflicts with activation={activation!r}")
            epi = self._ACT[activation]
        self.handle = gemm_plan_create(self.dab, self.dab, self.dcd, self.dcd, Dtype.F32,
                                       _LAYOUT[la], _LAYOUT[lb], _LAYOUT[lc], epi)

    def close(self):
        if self.handle:
            gemm_plan_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def set_config(self, schedule=Schedule.AUTO, tile=Tile.AUTO, sk_grid: int = 0):
        gemm_plan_set_config(self.handle, schedule, tile, sk_grid)
        return self

    def describe_batched(self, M, N, K, batch, num_cus=0) -> dict:
        return gemm_plan_describe_batched(self.handle, M, N, K, batch, num_cus)

    def describe(self, M, N, K, num_cus=0) -> dict:
        return gemm_plan_describe(self.handle, M, N, K, num_cus)

    def check(self, A, B, C, D, M, N, K, beta):
        if min(M, N, K) < 0:
            return   # the library reports negative sizes itself
        if M and N:
            _need(D, M * N, "D", self.dcd)
            if K:
                _need(A, M * K, "A", self.dab)
                _need(B, K * N, "B", self.dab)
            if beta != 0.0:
                _need(C, M * N, "C", self.dcd)

    def run(self, A, B, C, D, M, N, K, alpha=1.0, beta=0.0, scale_a=None, scale_b=None,
            stream=None, bias=None):
        self.check(A, B, C, D, M, N, K, beta)
        if bias is not None:
            if M and N:
                _need(bias, N, "bias", self.dcd)
            gemm_plan_run_ex(self.handle, A, B, C, D, bias, M, N, K, alpha, beta, scale_a,
                             scale_b, stream)
        elif scale_a is None and scale_b is None:
            gemm_plan_run(self.handle, A, B, C, D, M, N, K, alpha, beta, stream)
        else:
            gemm_plan_run_scaled(self.handle, A, B, C, D, M, N, K, alpha, beta, scale_a,
                                 scale_b, stream)

    def prepare(self, A, B, C, D, M, N, K, alpha=1.0, beta=0.0, stream=None) -> PreparedRun:
        """run(A, B, C, D, M, N, K, alpha, beta) checked and packed once; the
        returned PreparedRun launches it when called."""
        return PreparedRun(self, A, B, C, D, M, N, K, alpha, beta, stream)

    def run_noalloc(self, A, B, C, D, M, N, K, alpha=1.0, beta=0.0, stream=None):
        """gemm_plan_run_noalloc: run() without any device allocation (the
        stream-K / split-K workspace is the library's static one)."""
        self.check(A, B, C, D, M, N, K, beta)
        gemm_plan_run_noalloc(self.handle, A, B, C, D, M, N, K, alpha, beta, stream)

    def run_mx(self, A, B, C, D, M, N, K, mx_scale_a, mx_scale_b, alpha=1.0, beta=0.0,
               stream=None, bias=None):
        """MX block-scaled GEMM: mx_scale_a [M, K/32] and mx_scale_b [N, K/32]
        uint8 E8M0 device tensors."""
        import torch
        self.check(A, B, C, D, M, N, K, beta)
        if min(M, N, K) > 0 and K % 32 == 0:
            for t, rows, name in ((mx_scale_a, M, "mx_scale_a"), (mx_scale_b, N, "mx_scale_b")):
                if t is None or not t.is_cuda or t.dtype != torch.uint8 or not t.is_contiguous():
                    raise ValueError(f"{name} must be a contiguous uint8 device tensor")
                if t.numel() < rows * (K // 32):
                    raise ValueError(f"{name} holds {t.numel()} bytes, needs {rows * (K // 32)}")
            if bias is not None:
                _need(bias, N, "bias", self.dcd)
        gemm_plan_run_mx(self.handle, A, B, C, D, bias, M, N, K, alpha, beta, mx_scale_a,
                         mx_scale_b, stream)

    def run_aux(self, A, B, C, D, M, N, K, aux=None, aux_op="add", aux_pos="before",
                aux_out=None, alpha=1.0, beta=0.0, scale_a=None, scale_b=None, stream=None,
                bias=None):
        """Auxiliary-tensor epilogue: aux (M x N, C's type and layout) combined
        by aux_op ("add", "sub", "mul", "div") before or after the activation;
        aux_out (M x N, D's type and layout) receives the activation's input."""
        self.check(A, B, C, D, M, N, K, beta)
        if M and N:
            if bias is not None:
                _need(bias, N, "bias", self.dcd)
            if aux is not None:
                _need(aux, M * N, "aux", self.dcd)
            if aux_out is not None:
                _need(aux_out, M * N, "aux_out", self.dcd)
        op = AUX_OP[aux_op] if isinstance(aux_op, str) else int(aux_op)
        pos = AUX_POS[aux_pos] if isinstance(aux_pos, str) else int(aux_pos)
        gemm_plan_run_aux(self.handle, A, B, C, D, bias, aux, op, pos, aux_out, M, N, K, alpha,
                          beta, scale_a, scale_b, stream)

    def profile(self, A, B, C, D, M, N, K, alpha=1.0, beta=0.0, iters=10, stream=None):
        """Time every distinct launch for this shape (fastest first) and cache the best."""
        self.check(A, B, C, D, M, N, K, beta)
        return gemm_plan_profile(self.handle, A, B, C, D, M, N, K, alpha, beta, iters,
                                 stream=stream)

    def cache_export(self) -> str:
        return gemm_plan_cache_export(self.handle)

    def cache_import(self, text: str) -> None:
        gemm_plan_cache_import(self.handle, text)

    def cache_size(self) -> int:
        return gemm_plan_cache_size(self.handle)

    def cache_clear(self) -> None:
        gemm_plan_cache_clear(self.handle)

    def run_batched(self, A, B, C, D, M, N, K, batch, strides, alpha=1.0, beta=0.0,
                    scale_a=None, scale_b=None, stream=None, bias=None):
        """strides: (stride_a, stride_b, stride_c, stride_d) in elements."""
        sa, sb, sc, sd = (int(x) for x in strides)
        if min(M, N, K, batch, sa, sb, sc, sd) >= 0 and M and N and batch:
            last = batch - 1
            _need(D, last * sd + M * N, "D", self.dcd)
            if K:
                _need(A, last * sa + M * K, "A", self.dab)
                _need(B, last * sb + K * N, "B", self.dab)
            if beta != 0.0:
                _need(C, last * sc + M * N, "C", self.dcd)
            if bias is not None:
                _need(bias, N, "bias", self.dcd)
        gemm_plan_run_batched(self.handle, A, B, C, D, bias, M, N, K, batch, sa, sb, sc, sd,
                              alpha, beta, scale_a, scale_b, stream)

    def prepare_grouped(self, problems: Iterable[tuple], beta=0.0) -> "GroupedProblems":
        """Check a grouped problem list once and pack it into the C array
        grouped_gemm_run takes; run_grouped with the result skips both."""
        return GroupedProblems(self, problems, beta)

    def run_grouped(self, problems, alpha=1.0, beta=0.0, stream=None):
        """problems: a sequence of (M, N, K, A, B, C, D), or a GroupedProblems
        prepared by this plan (checked for a beta that reads C)."""
        if isinstance(problems, GroupedProblems):
            if problems.plan is not self:
                raise ValueError("GroupedProblems was prepared for another plan")
            if beta != 0.0 and problems.beta == 0.0:
                raise ValueError("GroupedProblems was prepared for beta == 0: C was not checked")
            _check(lib.grouped_gemm_run(self.handle, problems.arr, problems.count, alpha, beta,
                                        _stream(stream)))
            return
        probs = list(problems)
        for (M, N, K, A, B, C, D) in probs:
            self.check(A, B, C, D, M, N, K, beta)
        grouped_gemm_run(self.handle, probs, alpha, beta, stream)
