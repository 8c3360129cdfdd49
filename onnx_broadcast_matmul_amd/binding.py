"""ctypes binding of libmm.so (argument marshalling only).

Every computation runs in the HIP kernels behind the C ABI declared in
``include/mm.h``; this module converts shapes and torch tensors to the plain
pointers and sizes the ABI takes, and raises on error statuses.  There is no
fallback: if ``libmm.so`` is missing the first call raises.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional, Sequence, Tuple

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmm.so")

FLOAT, FLOAT16, DOUBLE, BFLOAT16 = 1, 10, 11, 16
UINT8, INT8, INT32 = 2, 3, 6
ZP_NONE, ZP_SCALAR, ZP_VECTOR = 0, 1, 2
MAX_BATCH_DIMS = 8
MAX_RANK = MAX_BATCH_DIMS + 2

ALGO_AUTO, ALGO_EMPTY, ALGO_ZERO_FILL, ALGO_DIRECT = 0, 1, 2, 3
ALGO_SKINNY_M, ALGO_SKINNY_N, ALGO_SPLIT_K, ALGO_GENERAL = 4, 5, 6, 7
ALGO_NAMES = {0: "auto", 1: "empty", 2: "zero_fill", 3: "direct", 4: "skinny_m", 5: "skinny_n",
              6: "split_k", 7: "general"}

ERR_NULL_ARG, ERR_RANK, ERR_NEG_DIM, ERR_K_MISMATCH, ERR_BROADCAST = 1, 2, 3, 4, 5
ERR_DTYPE, ERR_BAD_OPTION, ERR_TOO_LARGE, ERR_ALLOC, ERR_HIP = 6, 7, 8, 9, 10
ERR_SIZE, ERR_NO_CONSTANT_B = 11, 12


class MMError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"mm status {status}: {detail}")
        self.status = status
        self.detail = detail


class PlanOptions(ctypes.Structure):
    _fields_ = [("force_algo", ctypes.c_int32), ("tile", ctypes.c_int32), ("split_k", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class PlanInfo(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int32), ("algo", ctypes.c_int32),
        ("M", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64),
        ("batch", ctypes.c_int64), ("kernel_m", ctypes.c_int64),
        ("folded", ctypes.c_int32), ("batch_rank", ctypes.c_int32),
        ("batch_dims", ctypes.c_int64 * MAX_BATCH_DIMS),
        ("a_batch_strides", ctypes.c_int64 * MAX_BATCH_DIMS),
        ("b_batch_strides", ctypes.c_int64 * MAX_BATCH_DIMS),
        ("tile", ctypes.c_int32), ("split_k", ctypes.c_int32),
        ("k_chunk", ctypes.c_int64), ("workspace_bytes", ctypes.c_int64),
        ("flops", ctypes.c_double), ("min_bytes", ctypes.c_double),
        ("tail_col", ctypes.c_int64), ("tail_tile", ctypes.c_int32), ("constant_b_packed", ctypes.c_int32),
    ]


class GemmDesc(ctypes.Structure):
    _fields_ = [
        ("a_rows", ctypes.c_int64), ("a_cols", ctypes.c_int64),
        ("b_rows", ctypes.c_int64), ("b_cols", ctypes.c_int64),
        ("trans_a", ctypes.c_int32), ("trans_b", ctypes.c_int32),
        ("c_rank", ctypes.c_int32), ("reserved", ctypes.c_int32),
        ("c_shape", ctypes.c_int64 * 2),
        ("alpha", ctypes.c_float), ("beta", ctypes.c_float),
    ]


_lib = None
_lib_lock = threading.Lock()


def lib() -> ctypes.CDLL:
    """Load libmm.so (raises if it has not been built)."""
    global _lib
    with _lib_lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                               "or python -m onnx_broadcast_matmul_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        i64p = ctypes.POINTER(ctypes.c_int64)
        vp = ctypes.c_void_p
        L.mm_plan_create.argtypes = [i64p, ctypes.c_int, i64p, ctypes.c_int, ctypes.c_int, ctypes.POINTER(vp)]
        L.mm_plan_create.restype = ctypes.c_int
        L.mm_plan_create_ex.argtypes = [i64p, ctypes.c_int, i64p, ctypes.c_int, ctypes.c_int,
                                        ctypes.POINTER(PlanOptions), ctypes.POINTER(vp)]
        L.mm_plan_create_ex.restype = ctypes.c_int
        L.mm_plan_destroy.argtypes = [vp]
        L.mm_plan_destroy.restype = None
        L.mm_execute.argtypes = [vp, vp, vp, vp, vp]
        L.mm_execute.restype = ctypes.c_int
        L.mm_execute_noalloc.argtypes = [vp, vp, vp, vp, vp]
        L.mm_execute_noalloc.restype = ctypes.c_int
        L.mm_plan_output_shape.argtypes = [vp, i64p, ctypes.POINTER(ctypes.c_int)]
        L.mm_plan_output_shape.restype = ctypes.c_int
        L.mm_plan_output_numel.argtypes = [vp]
        L.mm_plan_output_numel.restype = ctypes.c_int64
        L.mm_plan_algo.argtypes = [vp]
        L.mm_plan_algo.restype = ctypes.c_int
        L.mm_plan_workspace_bytes.argtypes = [vp]
        L.mm_plan_workspace_bytes.restype = ctypes.c_size_t
        L.mm_plan_get_info.argtypes = [vp, ctypes.POINTER(PlanInfo)]
        L.mm_plan_get_info.restype = ctypes.c_int
        L.mm_tile_count.argtypes = [ctypes.c_int]
        L.mm_tile_count.restype = ctypes.c_int
        L.mm_tile_config.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_int),
                                     ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int)]
        L.mm_tile_config.restype = ctypes.c_int
        L.mm_plan_set_constant_b.argtypes = [vp, vp, ctypes.c_int64, vp]
        L.mm_plan_set_constant_b.restype = ctypes.c_int
        L.mm_plan_has_constant_b.argtypes = [vp]
        L.mm_plan_has_constant_b.restype = ctypes.c_int
        L.mm_execute_constant_b.argtypes = [vp, vp, vp, vp]
        L.mm_execute_constant_b.restype = ctypes.c_int
        L.mm_gemm_plan_create.argtypes = [ctypes.POINTER(GemmDesc), ctypes.c_int, ctypes.POINTER(PlanOptions),
                                           ctypes.POINTER(vp)]
        L.mm_gemm_plan_create.restype = ctypes.c_int
        L.mm_gemm_execute.argtypes = [vp, vp, vp, vp, vp, vp]
        L.mm_gemm_execute.restype = ctypes.c_int
        L.mm_int_plan_create.argtypes = [i64p, ctypes.c_int, i64p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_int, ctypes.c_int, ctypes.POINTER(PlanOptions), ctypes.POINTER(vp)]
        L.mm_int_plan_create.restype = ctypes.c_int
        L.mm_int_execute.argtypes = [vp, vp, vp, vp, vp, vp, vp]
        L.mm_int_execute.restype = ctypes.c_int
        L.mm_status_string.argtypes = [ctypes.c_int]
        L.mm_status_string.restype = ctypes.c_char_p
        L.mm_last_error.argtypes = []
        L.mm_last_error.restype = ctypes.c_char_p
        _lib = L
        return L


def _check(status: int) -> None:
    if status != 0:
        L = lib()
        detail = (L.mm_last_error() or b"").decode() or L.mm_status_string(status).decode()
        raise MMError(status, detail)


def _shape(shape: Sequence[int]):
    return (ctypes.c_int64 * max(1, len(shape)))(*[int(d) for d in shape])


def torch_dtype_code(dt) -> int:
    import torch

    codes = {torch.float32: FLOAT, torch.float16: FLOAT16, torch.bfloat16: BFLOAT16, torch.float64: DOUBLE}
    if dt not in codes:
        raise TypeError(f"unsupported tensor dtype {dt}")
    return codes[dt]


def torch_dtype(code: int):
    import torch

    return {FLOAT: torch.float32, FLOAT16: torch.float16, BFLOAT16: torch.bfloat16, DOUBLE: torch.float64,
            INT32: torch.int32, INT8: torch.int8, UINT8: torch.uint8}[code]


def tile_configs(dtype: int):
    L = lib()
    out = []
    for i in range(L.mm_tile_count(dtype)):
        bm, bn, bk = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
        _check(L.mm_tile_config(dtype, i, ctypes.byref(bm), ctypes.byref(bn), ctypes.byref(bk)))
        out.append((bm.value, bn.value, bk.value))
    return out


class Plan:
    """mm_plan_create / mm_execute / mm_plan_destroy for one (A shape, B shape, dtype)."""

    def __init__(self, a_shape: Sequence[int], b_shape: Sequence[int], dtype: int, force_algo: int = 0,
                 tile: int = 0, split_k: int = 0):
        L = lib()
        self._handle = ctypes.c_void_p()
        self.a_shape = tuple(int(d) for d in a_shape)
        self.b_shape = tuple(int(d) for d in b_shape)
        self.dtype = int(dtype)
        if force_algo or tile or split_k:
            opt = PlanOptions(force_algo, tile, split_k, 0)
            st = L.mm_plan_create_ex(_shape(self.a_shape), len(self.a_shape), _shape(self.b_shape),
                                     len(self.b_shape), self.dtype, ctypes.byref(opt), ctypes.byref(self._handle))
        else:
            st = L.mm_plan_create(_shape(self.a_shape), len(self.a_shape), _shape(self.b_shape),
                                  len(self.b_shape), self.dtype, ctypes.byref(self._handle))
        _check(st)
        self._lock = threading.Lock()

    def close(self) -> None:
        """mm_plan_destroy (the caller makes sure no execution is in flight)."""
        h = getattr(self, "_handle", None)
        if h is not None and h.value and _lib is not None:
            _lib.mm_plan_destroy(h)
            self._handle = ctypes.c_void_p()

    def __del__(self):
        self.close()

    @property
    def handle(self) -> ctypes.c_void_p:
        return self._handle

    @property
    def output_shape(self) -> Tuple[int, ...]:
        shp = (ctypes.c_int64 * MAX_RANK)()
        rank = ctypes.c_int()
        _check(lib().mm_plan_output_shape(self._handle, shp, ctypes.byref(rank)))
        return tuple(shp[i] for i in range(rank.value))

    @property
    def output_numel(self) -> int:
        return int(lib().mm_plan_output_numel(self._handle))

    @property
    def algo(self) -> int:
        return int(lib().mm_plan_algo(self._handle))

    @property
    def workspace_bytes(self) -> int:
        return int(lib().mm_plan_workspace_bytes(self._handle))

    def info(self) -> dict:
        inf = PlanInfo()
        _check(lib().mm_plan_get_info(self._handle, ctypes.byref(inf)))
        nb = inf.batch_rank
        return {
            "dtype": inf.dtype, "algo": inf.algo, "algo_name": ALGO_NAMES.get(inf.algo, "?"),
            "M": inf.M, "N": inf.N, "K": inf.K, "batch": inf.batch, "kernel_m": inf.kernel_m,
            "folded": bool(inf.folded), "batch_dims": tuple(inf.batch_dims[:nb]),
            "a_batch_strides": tuple(inf.a_batch_strides[:nb]), "b_batch_strides": tuple(inf.b_batch_strides[:nb]),
            "tile": inf.tile, "split_k": inf.split_k, "k_chunk": inf.k_chunk,
            "workspace_bytes": inf.workspace_bytes, "flops": inf.flops, "min_bytes": inf.min_bytes,
            "tail_col": inf.tail_col, "tail_tile": inf.tail_tile, "constant_b_packed": inf.constant_b_packed,
        }

    def execute_ptr(self, A: int, B: int, Y: int, stream: int = 0) -> None:
        """mm_execute on raw device pointers and a raw hipStream_t."""
        _check(lib().mm_execute(self._handle, ctypes.c_void_p(A), ctypes.c_void_p(B), ctypes.c_void_p(Y),
                                ctypes.c_void_p(stream)))

    def execute_noalloc_ptr(self, A: int, B: int, Y: int, stream: int = 0) -> None:
        """mm_execute_noalloc on raw device pointers and a raw hipStream_t."""
        _check(lib().mm_execute_noalloc(self._handle, ctypes.c_void_p(A), ctypes.c_void_p(B), ctypes.c_void_p(Y),
                                        ctypes.c_void_p(stream)))

    def execute_noalloc(self, A, B, Y, stream=None) -> None:
        """mm_execute_noalloc on torch device tensors (checked as in execute)."""
        self.execute(A, B, Y, stream, _entry=self.execute_noalloc_ptr)

    def execute(self, A, B, Y, stream=None, _entry=None) -> None:
        """mm_execute on torch device tensors; ``stream`` is a torch.cuda.Stream
        (default: the current stream of Y's device)."""
        import torch

        want = torch_dtype(self.dtype)
        for name, t, shape in (("A", A, self.a_shape), ("B", B, self.b_shape), ("Y", Y, self.output_shape)):
            if t.dtype != want:
                raise TypeError(f"{name} has dtype {t.dtype}, plan expects {want}")
            if tuple(t.shape) != tuple(shape):
                raise ValueError(f"{name} has shape {tuple(t.shape)}, plan expects {tuple(shape)}")
            if not t.is_contiguous():
                raise ValueError(f"{name} must be contiguous")
            if t.numel() and not t.is_cuda:
                raise ValueError(f"{name} must be a device tensor")
        if stream is None:
            stream = torch.cuda.current_stream(Y.device)
        with self._lock:
            (_entry or self.execute_ptr)(A.data_ptr(), B.data_ptr(), Y.data_ptr(), stream.cuda_stream)

    # ---- plan-owned constant B
    def set_constant_b_ptr(self, B: int, numel: int, stream: int = 0) -> None:
        """mm_plan_set_constant_b on a raw device pointer (copy completes before return)."""
        _check(lib().mm_plan_set_constant_b(self._handle, ctypes.c_void_p(B), ctypes.c_int64(numel),
                                            ctypes.c_void_p(stream)))

    def set_constant_b(self, B, stream=None) -> None:
        """Copy the device tensor B (the planned B shape and type) into plan-owned storage."""
        import torch

        if B.dtype != torch_dtype(self.dtype) or tuple(B.shape) != self.b_shape or not B.is_contiguous():
            raise ValueError(f"B must be a contiguous {torch_dtype(self.dtype)} tensor of shape {self.b_shape}")
        if stream is None:
            stream = torch.cuda.current_stream(B.device)
        with self._lock:
            self.set_constant_b_ptr(B.data_ptr(), B.numel(), stream.cuda_stream)

    @property
    def has_constant_b(self) -> bool:
        return bool(lib().mm_plan_has_constant_b(self._handle))

    def execute_constant_b_ptr(self, A: int, Y: int, stream: int = 0) -> None:
        """mm_execute_constant_b on raw device pointers."""
        _check(lib().mm_execute_constant_b(self._handle, ctypes.c_void_p(A), ctypes.c_void_p(Y),
                                           ctypes.c_void_p(stream)))

    def execute_constant_b(self, A, Y, stream=None) -> None:
        """mm_execute_constant_b on torch device tensors (B is the plan's own)."""
        import torch

        want = torch_dtype(self.dtype)
        for name, t, shape in (("A", A, self.a_shape), ("Y", Y, self.output_shape)):
            if t.dtype != want or tuple(t.shape) != tuple(shape) or not t.is_contiguous():
                raise ValueError(f"{name} must be a contiguous {want} tensor of shape {tuple(shape)}")
        if stream is None:
            stream = torch.cuda.current_stream(Y.device)
        with self._lock:
            self.execute_constant_b_ptr(A.data_ptr(), Y.data_ptr(), stream.cuda_stream)


class GemmPlan(Plan):
    """mm_gemm_plan_create / mm_gemm_execute: ONNX Gemm of rank-2 A, B with
    transA / transB, alpha, beta and an optional C broadcast to [M, N]."""

    def __init__(self, a_shape, b_shape, dtype: int, trans_a: bool = False, trans_b: bool = False,
                 c_shape=None, alpha: float = 1.0, beta: float = 1.0, force_algo: int = 0, tile: int = 0,
                 split_k: int = 0):
        L = lib()
        self._handle = ctypes.c_void_p()
        self.a_shape = tuple(int(d) for d in a_shape)
        self.b_shape = tuple(int(d) for d in b_shape)
        self.c_shape = None if c_shape is None else tuple(int(d) for d in c_shape)
        self.dtype = int(dtype)
        if len(self.a_shape) != 2 or len(self.b_shape) != 2:
            raise ValueError("Gemm takes rank-2 A and B")
        d = GemmDesc()
        d.a_rows, d.a_cols = self.a_shape
        d.b_rows, d.b_cols = self.b_shape
        d.trans_a, d.trans_b = int(trans_a), int(trans_b)
        d.c_rank = -1 if self.c_shape is None else len(self.c_shape)
        for i, v in enumerate(self.c_shape or ()):
            d.c_shape[i] = v
        d.alpha, d.beta = float(alpha), float(beta)
        opt = PlanOptions(force_algo, tile, split_k, 0)
        _check(L.mm_gemm_plan_create(ctypes.byref(d), self.dtype, ctypes.byref(opt), ctypes.byref(self._handle)))
        self._lock = threading.Lock()

    def execute_ptr(self, A: int, B: int, Y: int, stream: int = 0, C: int = 0) -> None:
        _check(lib().mm_gemm_execute(self._handle, ctypes.c_void_p(A), ctypes.c_void_p(B), ctypes.c_void_p(C),
                                     ctypes.c_void_p(Y), ctypes.c_void_p(stream)))

    def execute(self, A, B, Y, C=None, stream=None) -> None:
        import torch

        want = torch_dtype(self.dtype)
        checks = [("A", A, self.a_shape), ("B", B, self.b_shape), ("Y", Y, self.output_shape)]
        if self.c_shape is not None:
            if C is None:
                raise ValueError("this Gemm plan has a C")
            checks.append(("C", C, self.c_shape))
        for name, t, shape in checks:
            if t.dtype != want or tuple(t.shape) != tuple(shape) or not t.is_contiguous():
                raise ValueError(f"{name} must be a contiguous {want} tensor of shape {tuple(shape)}")
        if stream is None:
            stream = torch.cuda.current_stream(Y.device)
        with self._lock:
            self.execute_ptr(A.data_ptr(), B.data_ptr(), Y.data_ptr(), stream.cuda_stream,
                             C.data_ptr() if C is not None else 0)


def torch_int_code(dt) -> int:
    import torch

    codes = {torch.uint8: UINT8, torch.int8: INT8}
    if dt not in codes:
        raise TypeError(f"MatMulInteger takes uint8 / int8 tensors, not {dt}")
    return codes[dt]


class IntPlan(Plan):
    """mm_int_plan_create / mm_int_execute: ONNX MatMulInteger (UINT8 / INT8
    operands, optional scalar or per-row / per-column zero points, INT32
    output modulo 2^32)."""

    def __init__(self, a_shape, b_shape, a_type: int, b_type: int, a_zp: int = ZP_NONE, b_zp: int = ZP_NONE,
                 force_algo: int = 0, tile: int = 0, split_k: int = 0):
        L = lib()
        self._handle = ctypes.c_void_p()
        self.a_shape = tuple(int(d) for d in a_shape)
        self.b_shape = tuple(int(d) for d in b_shape)
        self.a_type, self.b_type = int(a_type), int(b_type)
        self.a_zp, self.b_zp = int(a_zp), int(b_zp)
        self.dtype = INT32
        opt = PlanOptions(force_algo, tile, split_k, 0)
        _check(L.mm_int_plan_create(_shape(self.a_shape), len(self.a_shape), _shape(self.b_shape), len(self.b_shape),
                                    self.a_type, self.b_type, self.a_zp, self.b_zp, ctypes.byref(opt),
                                    ctypes.byref(self._handle)))
        self._lock = threading.Lock()

    def zero_point_numel(self, which: str) -> int:
        """Elements the plan reads from the A or B zero point (0 for none)."""
        kind = self.a_zp if which == "a" else self.b_zp
        if kind == ZP_NONE:
            return 0
        if kind == ZP_SCALAR:
            return 1
        inf = self.info()
        return inf["M"] if which == "a" else inf["N"]

    def execute_ptr(self, A: int, B: int, Y: int, stream: int = 0, a_zp: int = 0, b_zp: int = 0) -> None:
        _check(lib().mm_int_execute(self._handle, ctypes.c_void_p(A), ctypes.c_void_p(B), ctypes.c_void_p(a_zp),
                                    ctypes.c_void_p(b_zp), ctypes.c_void_p(Y), ctypes.c_void_p(stream)))

    def execute(self, A, B, Y, a_zp=None, b_zp=None, stream=None) -> None:
        import torch

        tdt = {UINT8: torch.uint8, INT8: torch.int8}
        checks = [("A", A, self.a_shape, tdt[self.a_type]), ("B", B, self.b_shape, tdt[self.b_type]),
                  ("Y", Y, self.output_shape, torch.int32)]
        for which, zp, typ in (("a", a_zp, self.a_type), ("b", b_zp, self.b_type)):
            n = self.zero_point_numel(which)
            if (zp is None) != (n == 0):
                raise ValueError(f"{which}_zp: the plan expects {'none' if n == 0 else f'{n} value(s)'}")
            if zp is not None:
                if zp.numel() != n:
                    raise ValueError(f"{which}_zp has {zp.numel()} elements, the plan reads {n}")
                checks.append((f"{which}_zp", zp, tuple(zp.shape), tdt[typ]))
        for name, t, shape, want in checks:
            if t.dtype != want or tuple(t.shape) != tuple(shape) or not t.is_contiguous():
                raise ValueError(f"{name} must be a contiguous {want} tensor of shape {tuple(shape)}")
        if stream is None:
            stream = torch.cuda.current_stream(Y.device)
        with self._lock:
            self.execute_ptr(A.data_ptr(), B.data_ptr(), Y.data_ptr(), stream.cuda_stream,
                             a_zp.data_ptr() if a_zp is not None else 0, b_zp.data_ptr() if b_zp is not None else 0)


_plan_cache = {}
_plan_cache_lock = threading.Lock()


def matmul(A, B, out=None, stream=None):
    """Y = MatMul(A, B) (ONNX semantics) on ``stream`` (default: the current
    stream of A's device).  Plans are cached per (shapes, dtype, stream), so a
    plan's split-K workspace is never shared by two streams."""
    import torch

    code = torch_dtype_code(A.dtype)
    if B.dtype != A.dtype:
        raise TypeError(f"mixed input types {A.dtype} and {B.dtype}")
    if stream is None:
        stream = torch.cuda.current_stream(A.device)
    key = (tuple(A.shape), tuple(B.shape), code, A.device.index, stream.cuda_stream)
    with _plan_cache_lock:
        plan = _plan_cache.get(key)
        if plan is None:
            plan = Plan(A.shape, B.shape, code)
            _plan_cache[key] = plan
    if out is None:
        out = torch.empty(plan.output_shape, dtype=A.dtype, device=A.device)
    plan.execute(A, B, out, stream)
    return out
