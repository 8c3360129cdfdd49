"""CPU oracle for ONNX MatMul, Gemm and MatMulInteger -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never calls it and
shares no code with it.

The arithmetic lives in ``oracle.c`` (plain C, fp64 accumulation over an
explicit broadcast index walk; exact int64 sums for MatMulInteger); this module only builds it with gcc and
marshals numpy arrays through ctypes.  ``compare.py`` holds the comparator
that applies the parity tolerances.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

# ONNX TensorProto type codes.
FLOAT, FLOAT16, DOUBLE, BFLOAT16 = 1, 10, 11, 16

STATUS = {
    0: "ok",
    1: "rank",
    2: "negative dimension",
    3: "inner dimension mismatch",
    4: "batch dimensions not broadcastable",
    5: "unknown dtype",
    6: "allocation failed",
    7: "Gemm operand shapes or zero-point kinds do not fit",
}


class OracleError(RuntimeError):
    def __init__(self, code: int):
        super().__init__(f"oracle status {code}: {STATUS.get(code, '?')}")
        self.code = code


def build() -> str:
    """Compile oracle.c into liboracle.so with gcc (always recompiles)."""
    cmd = [
        "gcc", "-O2", "-ftree-vectorize", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared",
        "-Wall", "-Wextra", SRC, "-o", LIB + ".tmp", "-lm",
    ]
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        L = ctypes.CDLL(LIB)
        i64p = ctypes.POINTER(ctypes.c_int64)
        L.oracle_output_shape.argtypes = [i64p, ctypes.c_int, i64p, ctypes.c_int, i64p,
                                          ctypes.POINTER(ctypes.c_int)]
        L.oracle_matmul.argtypes = [ctypes.c_int, ctypes.c_void_p, i64p, ctypes.c_int,
                                    ctypes.c_void_p, i64p, ctypes.c_int, ctypes.c_void_p]
        L.oracle_matmul_at.argtypes = [ctypes.c_int, ctypes.c_void_p, i64p, ctypes.c_int,
                                       ctypes.c_void_p, i64p, ctypes.c_int, ctypes.c_void_p,
                                       ctypes.c_int64, ctypes.c_void_p]
        L.oracle_narrow_array.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int64,
                                          ctypes.c_void_p]
        L.oracle_decode_array.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int64,
                                          ctypes.c_void_p]
        L.oracle_narrow_f16.argtypes = [ctypes.c_double]
        L.oracle_narrow_f16.restype = ctypes.c_uint16
        L.oracle_narrow_bf16.argtypes = [ctypes.c_double]
        L.oracle_narrow_bf16.restype = ctypes.c_uint16
        L.oracle_decode_f16.argtypes = [ctypes.c_uint16]
        L.oracle_decode_f16.restype = ctypes.c_double
        L.oracle_decode_bf16.argtypes = [ctypes.c_uint16]
        L.oracle_decode_bf16.restype = ctypes.c_double
        L.oracle_threads.restype = ctypes.c_int
        L.oracle_gemm.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                                  ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p,
                                  i64p, ctypes.c_int, ctypes.c_double, ctypes.c_double, ctypes.c_void_p]
        L.oracle_gemm_at.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                                     ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                                     ctypes.c_void_p, i64p, ctypes.c_int, ctypes.c_double, ctypes.c_double,
                                     ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
        int_args = [ctypes.c_void_p, i64p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, i64p, ctypes.c_int,
                    ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_int]
        L.oracle_matmul_integer.argtypes = int_args + [ctypes.c_void_p]
        L.oracle_matmul_integer_at.argtypes = int_args + [i64p, ctypes.c_int64, ctypes.c_void_p]
        _lib = L
    return _lib


def _shape_arr(shape):
    arr = (ctypes.c_int64 * max(1, len(shape)))(*[int(d) for d in shape])
    return arr


def _storage(x: np.ndarray, dtype: int) -> np.ndarray:
    """Contiguous raw storage: float32, float64, or uint16 bit patterns."""
    want = {FLOAT: np.float32, DOUBLE: np.float64, FLOAT16: np.uint16, BFLOAT16: np.uint16}[dtype]
    if x.dtype == np.float16 and dtype == FLOAT16:
        x = x.view(np.uint16)
    if x.dtype != want:
        raise TypeError(f"storage for dtype {dtype} must be {want}, got {x.dtype}")
    return np.ascontiguousarray(x)


def output_shape(a_shape, b_shape):
    """Output shape of MatMul(A, B); raises OracleError on invalid shapes."""
    out = (ctypes.c_int64 * (max(len(a_shape), len(b_shape)) + 1))()
    rank = ctypes.c_int(0)
    st = lib().oracle_output_shape(_shape_arr(a_shape), len(a_shape), _shape_arr(b_shape),
                                   len(b_shape), out, ctypes.byref(rank))
    if st:
        raise OracleError(st)
    return tuple(out[i] for i in range(rank.value))


def matmul(a: np.ndarray, b: np.ndarray, dtype: int) -> np.ndarray:
    """Exact-to-fp64 MatMul of stored tensors ``a`` and ``b`` (raw storage:
    float32 / float64 arrays, or uint16 bit patterns for FLOAT16/BFLOAT16).
    Returns a float64 array of the output shape."""
    a = _storage(a, dtype)
    b = _storage(b, dtype)
    shape = output_shape(a.shape, b.shape)
    y = np.empty(int(np.prod(shape, dtype=np.int64)), dtype=np.float64)
    st = lib().oracle_matmul(dtype, a.ctypes.data, _shape_arr(a.shape), a.ndim, b.ctypes.data,
                             _shape_arr(b.shape), b.ndim, y.ctypes.data)
    if st:
        raise OracleError(st)
    return y.reshape(shape)


def matmul_at(a: np.ndarray, b: np.ndarray, dtype: int, flat_idx) -> np.ndarray:
    """Selected outputs (flat row-major indices into the output) as float64."""
    a = _storage(a, dtype)
    b = _storage(b, dtype)
    idx = np.ascontiguousarray(np.asarray(flat_idx, dtype=np.int64))
    out = np.empty(idx.size, dtype=np.float64)
    st = lib().oracle_matmul_at(dtype, a.ctypes.data, _shape_arr(a.shape), a.ndim,
                                b.ctypes.data, _shape_arr(b.shape), b.ndim, idx.ctypes.data,
                                idx.size, out.ctypes.data)
    if st:
        raise OracleError(st)
    return out


def narrow(x: np.ndarray, dtype: int) -> np.ndarray:
    """Round float64 values to the storage of ``dtype`` (nearest, ties to even).
    Returns float32 / float64 arrays, or uint16 bit patterns for 16-bit types."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    out_dt = {FLOAT: np.float32, DOUBLE: np.float64, FLOAT16: np.uint16, BFLOAT16: np.uint16}[dtype]
    out = np.empty(x.shape, dtype=out_dt)
    st = lib().oracle_narrow_array(dtype, x.ctypes.data, x.size, out.ctypes.data)
    if st:
        raise OracleError(st)
    return out


def decode(bits: np.ndarray, dtype: int) -> np.ndarray:
    """Exact float64 values of stored elements."""
    bits = _storage(np.asarray(bits), dtype)
    out = np.empty(bits.shape, dtype=np.float64)
    st = lib().oracle_decode_array(dtype, bits.ctypes.data, bits.size, out.ctypes.data)
    if st:
        raise OracleError(st)
    return out


def gemm(a: np.ndarray, b: np.ndarray, dtype: int, trans_a: bool = False, trans_b: bool = False,
         c: np.ndarray = None, alpha: float = 1.0, beta: float = 1.0) -> np.ndarray:
    """ONNX Gemm of stored rank-2 tensors (raw storage as for ``matmul``):
    alpha * A' B' + beta * C, with C (optional) broadcast to [M, N].  alpha
    and beta are taken as given (float64).  Returns float64 [M, N]."""
    a = _storage(a, dtype)
    b = _storage(b, dtype)
    if a.ndim != 2 or b.ndim != 2:
        raise OracleError(7)
    M = a.shape[1] if trans_a else a.shape[0]
    N = b.shape[0] if trans_b else b.shape[1]
    y = np.empty(M * N, dtype=np.float64)
    cptr, cshape, crank = None, _shape_arr(()), -1
    if c is not None:
        c = _storage(c, dtype)
        cptr, cshape, crank = c.ctypes.data, _shape_arr(c.shape), c.ndim
    st = lib().oracle_gemm(dtype, a.ctypes.data, a.shape[0], a.shape[1], int(trans_a), b.ctypes.data,
                           b.shape[0], b.shape[1], int(trans_b), cptr, cshape, crank, float(alpha), float(beta),
                           y.ctypes.data)
    if st:
        raise OracleError(st)
    return y.reshape(M, N)


def gemm_at(a: np.ndarray, b: np.ndarray, dtype: int, flat_idx, trans_a: bool = False, trans_b: bool = False,
            c: np.ndarray = None, alpha: float = 1.0, beta: float = 1.0) -> np.ndarray:
    """Selected Gemm outputs (flat row-major indices into [M, N]) as float64."""
    a = _storage(a, dtype)
    b = _storage(b, dtype)
    if a.ndim != 2 or b.ndim != 2:
        raise OracleError(7)
    idx = np.ascontiguousarray(np.asarray(flat_idx, dtype=np.int64))
    out = np.empty(idx.size, dtype=np.float64)
    cptr, cshape, crank = None, _shape_arr(()), -1
    if c is not None:
        c = _storage(c, dtype)
        cptr, cshape, crank = c.ctypes.data, _shape_arr(c.shape), c.ndim
    st = lib().oracle_gemm_at(dtype, a.ctypes.data, a.shape[0], a.shape[1], int(trans_a), b.ctypes.data,
                              b.shape[0], b.shape[1], int(trans_b), cptr, cshape, crank, float(alpha), float(beta),
                              idx.ctypes.data, idx.size, out.ctypes.data)
    if st:
        raise OracleError(st)
    return out


def _int_operand(x: np.ndarray):
    x = np.ascontiguousarray(x)
    if x.dtype not in (np.uint8, np.int8):
        raise TypeError(f"MatMulInteger operands are uint8 / int8, got {x.dtype}")
    return x, int(x.dtype == np.int8)


def _int_zero_point(zp, operand_dtype):
    """(pointer, kind, keep-alive array): kind 0 none, 1 scalar (0-d), 2
    vector (1-d)."""
    if zp is None:
        return None, 0, None
    zp = np.array(zp, dtype=operand_dtype, copy=True)  # keeps a 0-d value 0-d
    kind = 1 if zp.ndim == 0 else 2
    return zp.ctypes.data, kind, zp


def _int_call(a, b, za, zb, flat_idx):
    a, a_signed = _int_operand(a)
    b, b_signed = _int_operand(b)
    pza, kza, za = _int_zero_point(za, a.dtype)
    pzb, kzb, zb = _int_zero_point(zb, b.dtype)
    if kza == 2 and za.size != (1 if a.ndim == 1 else a.shape[-2]):
        raise ValueError("A zero-point vector must have one entry per row")
    if kzb == 2 and zb.size != (1 if b.ndim == 1 else b.shape[-1]):
        raise ValueError("B zero-point vector must have one entry per column")
    args = [a.ctypes.data, _shape_arr(a.shape), a.ndim, a_signed, b.ctypes.data, _shape_arr(b.shape), b.ndim,
            b_signed, pza, kza, pzb, kzb]
    if flat_idx is None:
        shape = output_shape(a.shape, b.shape)
        y = np.empty(int(np.prod(shape, dtype=np.int64)), dtype=np.int32)
        st = lib().oracle_matmul_integer(*args, y.ctypes.data)
        if st:
            raise OracleError(st)
        return y.reshape(shape)
    idx = np.ascontiguousarray(np.asarray(flat_idx, dtype=np.int64))
    out = np.empty(idx.size, dtype=np.int32)
    st = lib().oracle_matmul_integer_at(*args, idx.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), idx.size,
                                        out.ctypes.data)
    if st:
        raise OracleError(st)
    return out


def matmul_integer(a: np.ndarray, b: np.ndarray, a_zero_point=None, b_zero_point=None) -> np.ndarray:
    """ONNX MatMulInteger of uint8 / int8 arrays: the exact sum of
    (a - za)(b - zb) reduced modulo 2^32, as int32 of the output shape.  A
    zero point is None, a 0-d value, or a 1-d vector (A: one per row, B: one
    per column)."""
    return _int_call(a, b, a_zero_point, b_zero_point, None)


def matmul_integer_at(a, b, flat_idx, a_zero_point=None, b_zero_point=None) -> np.ndarray:
    """Selected MatMulInteger outputs (flat row-major indices) as int32."""
    return _int_call(a, b, a_zero_point, b_zero_point, flat_idx)


def threads() -> int:
    return int(lib().oracle_threads())
