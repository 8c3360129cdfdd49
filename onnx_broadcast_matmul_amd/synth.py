"""Seeded synthetic inputs for ONNX MatMul workloads.

This module only draws random numbers and stores them in the element type;
it holds none of the matrix-product arithmetic.  Both the GPU path (tests,
benchmark) and the CPU oracle consume exactly the bit patterns it returns.

Recipe: numpy ``default_rng`` (PCG64) seeded with ``[seed, product, operand]``
draws float32 values (float64 values for DOUBLE, so that their products do
not fit a double exactly) in fixed chunks of ``CHUNK`` elements; uniform(lo,
hi) is ``lo + (hi - lo) * U[0,1)``, normal(0, s) is ``s * N(0,1)``; "int"
draws integers uniformly from {-2, ..., 2}.  The float32 values are then
rounded to the element type: FLOAT16 by numpy's float32->float16 conversion,
BFLOAT16 by torch's float32->bfloat16 conversion (both round to nearest, ties
to even).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Sequence, Tuple

import numpy as np

FLOAT, FLOAT16, DOUBLE, BFLOAT16 = 1, 10, 11, 16
DTYPE_NAMES = {FLOAT: "fp32", FLOAT16: "fp16", DOUBLE: "fp64", BFLOAT16: "bf16"}
ELEM_SIZE = {FLOAT: 4, FLOAT16: 2, DOUBLE: 8, BFLOAT16: 2}
CHUNK = 1 << 24


def _draw(rng: np.random.Generator, n: int, dist: Tuple, ft=np.float32) -> np.ndarray:
    out = np.empty(n, dtype=ft)
    kind = dist[0]
    for s in range(0, n, CHUNK):
        e = min(n, s + CHUNK)
        if kind == "uniform":
            lo, hi = dist[1], dist[2]
            out[s:e] = rng.random(e - s, dtype=ft)
            out[s:e] *= ft(hi - lo)
            out[s:e] += ft(lo)
        elif kind == "normal":
            out[s:e] = rng.standard_normal(e - s, dtype=ft)
            out[s:e] *= ft(dist[1])
        elif kind == "int":
            out[s:e] = rng.integers(-2, 3, e - s).astype(ft)
        else:
            raise ValueError(f"unknown distribution {dist}")
    return out


def to_storage(x32: np.ndarray, dtype: int) -> np.ndarray:
    """float32 values (float64 for DOUBLE) -> element storage (float32,
    float64, or uint16 bit patterns)."""
    if dtype == FLOAT or dtype == DOUBLE:
        return x32
    if dtype == FLOAT16:
        return x32.astype(np.float16).view(np.uint16)
    if dtype == BFLOAT16:
        import torch

        out = np.empty(x32.shape, dtype=np.uint16)
        flat_in = x32.reshape(-1)
        flat_out = out.reshape(-1)
        for s in range(0, flat_in.size, CHUNK):
            e = min(flat_in.size, s + CHUNK)
            t = torch.from_numpy(flat_in[s:e]).to(torch.bfloat16)
            flat_out[s:e] = t.view(torch.int16).numpy().view(np.uint16)
        return out
    raise ValueError(f"dtype {dtype}")


def generate(shape: Sequence[int], dtype: int, dist: Tuple, seed: Sequence[int]) -> np.ndarray:
    """Storage array (float32, float64, or uint16 bits for 16-bit types) of ``shape``."""
    n = int(np.prod(shape, dtype=np.int64)) if len(shape) else 1
    rng = np.random.default_rng(list(seed))
    ft = np.float64 if dtype == DOUBLE else np.float32
    return to_storage(_draw(rng, n, dist, ft), dtype).reshape(tuple(shape))


def generate_scaled_int(shape: Sequence[int], dtype: int, seed: Sequence[int], ints: Tuple[int, int],
                        exps: Tuple[int, int], operand: str) -> np.ndarray:
    """Storage array of ``shape`` whose values are i * 2^e: integers i uniform
    over [ints[0], ints[1]] and exponents e uniform over [exps[0], exps[1]],
    one exponent per row of an A operand (``operand="a"``: shared along the
    last axis) or per column of a B operand (``operand="b"``: shared along
    the second-to-last axis).  Every value is exactly representable in the
    element type (checked); products of such operands are exact in FP32, and
    with |i| small their sums are too, so results can be steered past a
    type's largest finite value, into FP16 subnormals, or onto rounding ties
    while staying bit-for-bit determined."""
    shape = tuple(int(d) for d in shape)
    rng = np.random.default_rng(list(seed))
    n = int(np.prod(shape, dtype=np.int64)) if len(shape) else 1
    iv = rng.integers(ints[0], ints[1] + 1, n).astype(np.float64).reshape(shape)
    if len(shape) == 1:
        eshape = (1,) if operand == "a" else shape
    elif operand == "a":
        eshape = shape[:-1] + (1,)
    else:
        eshape = shape[:-2] + (1,) + shape[-1:]
    ev = rng.integers(exps[0], exps[1] + 1, int(np.prod(eshape, dtype=np.int64))).reshape(eshape)
    x = np.ldexp(iv, ev)
    ft = np.float64 if dtype == DOUBLE else np.float32
    x32 = x.astype(ft)
    if not np.array_equal(x32.astype(np.float64), x):
        raise ValueError("scaled integers must be exact in the staging type")
    st = to_storage(x32, dtype)
    if dtype == FLOAT16:
        back = st.view(np.float16).astype(np.float64)
    elif dtype == BFLOAT16:
        back = (st.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    else:
        back = st.astype(np.float64)
    if not np.array_equal(back, x):
        raise ValueError("scaled integers must be exact in the element type")
    return st


def as_torch(storage: np.ndarray, dtype: int):
    """CPU torch tensor viewing the same bits with the element type."""
    import torch

    shape = np.shape(storage)  # ascontiguousarray turns a 0-d array into 1-d
    if dtype == FLOAT or dtype == DOUBLE:
        return torch.from_numpy(np.ascontiguousarray(storage)).reshape(shape)
    t = torch.from_numpy(np.ascontiguousarray(storage).view(np.int16)).reshape(shape)
    return t.view(torch.float16 if dtype == FLOAT16 else torch.bfloat16)


def from_torch(t) -> np.ndarray:
    """Storage array of a (CPU or device) torch tensor."""
    import torch

    t = t.detach().cpu().contiguous()
    if t.dtype in (torch.float32, torch.float64):
        return t.numpy()
    return t.view(torch.int16).numpy().view(np.uint16)


@dataclass
class Product:
    """One MatMul: shapes, element type, value distribution and seed."""

    name: str
    a_shape: Tuple[int, ...]
    b_shape: Tuple[int, ...]
    dtype: int
    dist: Tuple
    seed: int
    index: int = 0

    @property
    def K(self) -> int:
        return int(self.a_shape[-1])

    def make(self, dist: Tuple = None) -> Tuple[np.ndarray, np.ndarray]:
        d = dist if dist is not None else self.dist
        a = generate(self.a_shape, self.dtype, d, [self.seed, self.index, 0])
        b = generate(self.b_shape, self.dtype, d, [self.seed, self.index, 1])
        return a, b


@dataclass
class Workload:
    name: str
    products: List[Product] = field(default_factory=list)


def _normal_over_sqrt_k(k: int) -> Tuple:
    return ("normal", 1.0 / math.sqrt(k))


def _workloads() -> dict:
    w = {}
    u1 = ("uniform", -1.0, 1.0)
    w["fp32_tiny_broadcast"] = Workload("fp32_tiny_broadcast", [
        Product("fp32_4x64x96_by_96x80", (4, 64, 96), (96, 80), FLOAT, u1, 1, 0),
        Product("fp32_vec96_by_96x80", (96,), (96, 80), FLOAT, u1, 1, 1),
        Product("fp32_4x64x96_by_vec96", (4, 64, 96), (96,), FLOAT, u1, 1, 2),
    ])
    w["fp32_square_and_batched_broadcast"] = Workload("fp32_square_and_batched_broadcast", [
        Product("fp32_1024_square", (1024, 1024), (1024, 1024), FLOAT, _normal_over_sqrt_k(1024), 2, 0),
        Product("fp32_8x1x512x512_by_1x6x512x512", (8, 1, 512, 512), (1, 6, 512, 512), FLOAT,
                _normal_over_sqrt_k(512), 2, 1),
    ])
    w["bf16_transformer_projection"] = Workload("bf16_transformer_projection", [
        Product("bf16_16x512x4096_by_4096x11008", (16, 512, 4096), (4096, 11008), BFLOAT16,
                ("normal", 0.02), 3, 0),
    ])
    u5 = ("uniform", -0.5, 0.5)
    w["fp16_decode_skinny"] = Workload("fp16_decode_skinny", [
        Product("fp16_gemv_32x1x4096_by_32x4096x4096", (32, 1, 4096), (32, 4096, 4096), FLOAT16, u5, 4, 0),
        Product("fp16_skinny_n_8192x4096_by_4096x8", (8192, 4096), (4096, 8), FLOAT16, u5, 4, 1),
    ])
    w["longk_and_attention"] = Workload("longk_and_attention", [
        Product("fp32_splitk_64x131072_by_131072x64", (64, 131072), (131072, 64), FLOAT,
                _normal_over_sqrt_k(131072), 5, 0),
        Product("bf16_qk_4x32x2048x128_by_4x32x128x2048", (4, 32, 2048, 128), (4, 32, 128, 2048), BFLOAT16,
                _normal_over_sqrt_k(128), 5, 1),
        Product("bf16_pv_4x32x2048x2048_by_4x32x2048x128", (4, 32, 2048, 2048), (4, 32, 2048, 128), BFLOAT16,
                _normal_over_sqrt_k(2048), 5, 2),
    ])
    # DOUBLE: the square and batch-broadcast shapes again, in FP64.
    w["fp64_square_and_batched_broadcast"] = Workload("fp64_square_and_batched_broadcast", [
        Product("fp64_1024_square", (1024, 1024), (1024, 1024), DOUBLE, _normal_over_sqrt_k(1024), 6, 0),
        Product("fp64_8x1x512x512_by_1x6x512x512", (8, 1, 512, 512), (1, 6, 512, 512), DOUBLE,
                _normal_over_sqrt_k(512), 6, 1),
    ])
    return w


WORKLOADS = _workloads()


@dataclass
class GemmProduct:
    """One ONNX Gemm: Y = alpha * A'B' + beta * C with A' = A or A^T
    (stored [K, M]), B' = B or B^T (stored [N, K]) and C of ``c_shape``."""

    name: str
    M: int
    N: int
    K: int
    trans_a: bool
    trans_b: bool
    c_shape: Tuple[int, ...]
    alpha: float
    beta: float
    dtype: int
    dist: Tuple
    seed: int

    @property
    def a_shape(self) -> Tuple[int, ...]:
        return (self.K, self.M) if self.trans_a else (self.M, self.K)

    @property
    def b_shape(self) -> Tuple[int, ...]:
        return (self.N, self.K) if self.trans_b else (self.K, self.N)

    def make(self):
        a = generate(self.a_shape, self.dtype, self.dist, [self.seed, 0, 0])
        b = generate(self.b_shape, self.dtype, self.dist, [self.seed, 0, 1])
        c = None if self.c_shape is None else generate(self.c_shape, self.dtype, self.dist, [self.seed, 0, 2])
        return a, b, c


# Gemm: the transformer projection as a linear layer, X W^T + bias, with the
# weight stored [N, K] as such layers keep it.
GEMM_PRODUCTS = [
    GemmProduct("bf16_linear_8192x4096_by_11008x4096T_bias", 8192, 11008, 4096, False, True, (11008,), 1.0, 1.0,
                BFLOAT16, ("normal", 0.02), 7),
]


def generate_int(shape: Sequence[int], signed: bool, seed: Sequence[int], lo: int = None, hi: int = None) -> np.ndarray:
    """int8 (signed) or uint8 array of ``shape``, uniform over [lo, hi]
    (default: the whole type range)."""
    lo = (-128 if signed else 0) if lo is None else lo
    hi = (127 if signed else 255) if hi is None else hi
    n = int(np.prod(shape, dtype=np.int64)) if len(shape) else 1
    rng = np.random.default_rng(list(seed))
    v = rng.integers(lo, hi + 1, size=n, dtype=np.int16)
    return v.astype(np.int8 if signed else np.uint8).reshape(tuple(shape))


@dataclass
class IntProduct:
    """One MatMulInteger: shapes, operand signedness, zero-point kinds
    (0 none, 1 scalar, 2 per row of A / per column of B) and seed; operands
    uniform over their whole type range."""

    name: str
    a_shape: Tuple[int, ...]
    b_shape: Tuple[int, ...]
    a_signed: bool
    b_signed: bool
    a_zp: int
    b_zp: int
    seed: int

    def make(self):
        a = generate_int(self.a_shape, self.a_signed, [self.seed, 0, 0])
        b = generate_int(self.b_shape, self.b_signed, [self.seed, 0, 1])
        m = 1 if len(self.a_shape) == 1 else self.a_shape[-2]
        n = 1 if len(self.b_shape) == 1 else self.b_shape[-1]
        za = None if self.a_zp == 0 else generate_int(() if self.a_zp == 1 else (m,), self.a_signed, [self.seed, 0, 2])
        zb = None if self.b_zp == 0 else generate_int(() if self.b_zp == 1 else (n,), self.b_signed, [self.seed, 0, 3])
        return a, b, za, zb


# MatMulInteger: the transformer projection quantized as the pages' integer
# benchmark quantizes it -- UINT8 activations with one zero point, INT8
# weights without one.
INT_PRODUCTS = [
    IntProduct("u8s8_16x512x4096_by_4096x11008", (16, 512, 4096), (4096, 11008), False, True, 1, 0, 9),
]


def all_products() -> List[Product]:
    return [p for w in WORKLOADS.values() for p in w.products]
