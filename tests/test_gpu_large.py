"""Operands and outputs past 4 GiB, one case per kernel family.

The kernels address memory with 64-bit element offsets (batch offsets, tile
origins, row pitches); the tiled kernels keep 32-bit buffer offsets inside
one tile's rows and hand a tile whose rows span 2 GiB or more to the
register-staged kernel.  Each case below puts an operand, or the output,
beyond 2^32 bytes for one algorithm: skinny-M (with its K split), both
skinny-N kernels, the tiled kernel over a broadcast batch with last-round
balancing, the persistent tiles and the one-tile kernel writing a 5 GiB
output, split-K whose 64-row tiles of A span 2 GiB (the register-staged
kernel), DOUBLE, and MatMulInteger.

Inputs are a seeded pattern of P values repeated over the flat storage of
each operand.  P is prime, so an offset that wraps or is truncated to 32
bits reads a different value.  Floating-point values are -1, 0 or 1, so
every FP32 partial sum is an exact integer below 2^24 and the outputs are
compared bit for bit with the oracle's values rounded once to the output
type.  The oracle receives the needed rows of A and columns of B, rebuilt
on the host from the same pattern, and computes the sampled outputs (first
and last rows and columns among them) from the definition.
"""
import numpy as np
import pytest

import oracle
from oracle.compare import check
from onnx_broadcast_matmul_amd import binding as mm
from onnx_broadcast_matmul_amd import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

P = 1_000_003  # pattern period (prime)
FOUR_GIB = 1 << 32


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    mm.lib()  # the native library must load: no fallback exists
    yield torch.device("cuda:0")
    torch.cuda.empty_cache()


def _pattern(dt, seed, signed=None):
    if dt is None:  # MatMulInteger operand
        return synth.generate_int((P,), signed, seed)
    return synth.generate_scaled_int((P,), dt, seed, (-1, 1), (0, 0), "a")


def _device(pattern, dt, shape, dev):
    """The pattern repeated over prod(shape) elements, on the device."""
    n = int(np.prod(shape, dtype=np.int64))
    t = torch.from_numpy(pattern) if dt is None else synth.as_torch(pattern, dt)
    return t.to(dev).repeat(-(-n // P))[:n].view(shape)


def _rows(pattern, shape, prefix, rows):
    """Rows `rows` of matrix `prefix` of a row-major operand of `shape`, as [len(rows), shape[-1]]."""
    base = int(np.ravel_multi_index(tuple(prefix) + (0, 0), shape)) if len(shape) > 1 else 0
    n = shape[-1]
    ar = np.arange(n, dtype=np.int64)
    return np.stack([pattern[(base + int(r) * n + ar) % P] for r in rows])


def _cols(pattern, shape, prefix, cols):
    """Columns `cols` of matrix `prefix` of a row-major operand of `shape`, as [shape[-2], len(cols)]."""
    base = int(np.ravel_multi_index(tuple(prefix) + (0, 0), shape))
    k, n = shape[-2], shape[-1]
    ar = np.arange(k, dtype=np.int64) * n
    return np.stack([pattern[(base + ar + int(c)) % P] for c in cols], axis=1)


def _pick(n, extra, rng):
    """First, last and a few random indices below n, plus `extra`."""
    v = np.concatenate([[0, n - 1], rng.integers(0, n, 6), np.asarray(extra, dtype=np.int64)])
    return np.unique(v[(v >= 0) & (v < n)])


def _nbytes(shape, dt):
    return int(np.prod(shape, dtype=np.int64)) * synth.ELEM_SIZE[dt]


CASES = [
    # (id, A shape, B shape, element type, algorithm the plan must take, what passes 4 GiB)
    ("skinny_m-fp16-B", (1, 32768), (32768, 70000), mm.FLOAT16, "skinny_m", "b"),
    ("skinny_n8-bf16-A", (600000, 4096), (4096, 8), mm.BFLOAT16, "skinny_n", "a"),
    ("skinny_n-fp16-A", (300000, 8192), (8192, 3), mm.FLOAT16, "skinny_n", "a"),
    ("general-bf16-broadcast-B", (2, 1, 256, 8192), (1, 3, 8192, 100000), mm.BFLOAT16, "general", "b"),
    ("general-persistent-bf16-Y", (65536, 64), (64, 40960), mm.BFLOAT16, "general", "y"),
    ("general-fp16-Y", (65536, 64), (64, 40000), mm.FLOAT16, "general", "y"),
    ("split_k-fp32-2GiB-rows", (64, 8388608), (8388608, 64), mm.FLOAT, "split_k", "span"),
    ("general-fp64-B", (64, 4096), (4096, 140000), mm.DOUBLE, "general", "b"),
]


@pytest.mark.parametrize("sa,sb,dt,want,big", [pytest.param(*c[1:], id=c[0]) for c in CASES])
def test_beyond_4gib(sa, sb, dt, want, big, dev):
    plan = mm.Plan(sa, sb, dt)
    inf = plan.info()
    assert mm.ALGO_NAMES[plan.algo] == want, inf
    out_shape = plan.output_shape
    if big == "a":
        assert _nbytes(sa, dt) > FOUR_GIB
    elif big == "b":
        assert _nbytes(sb, dt) > FOUR_GIB
    elif big == "y":
        assert _nbytes(out_shape, dt) > FOUR_GIB
        if sb[-1] % 256 == 0:
            assert inf["tile"] == 11  # the persistent kernel
    else:
        # the rows of one 64-row tile of A span 2 GiB: the register-staged kernel
        assert 64 * sa[-1] * synth.ELEM_SIZE[dt] >= (1 << 31) and inf["split_k"] > 1
    pa, pb = _pattern(dt, [77, 0]), _pattern(dt, [77, 1])
    A = _device(pa, dt, sa, dev)
    B = _device(pb, dt, sb, dev)
    Y = torch.full(out_shape, float("nan"), dtype=mm.torch_dtype(dt), device=dev)
    plan.execute(A, B, Y)
    torch.cuda.synchronize()
    del A, B

    rng = np.random.default_rng(5)
    K = sa[-1]
    M, N = sa[-2], sb[-1]
    # batch index pairs: the first and the last output matrix
    batch_shape = out_shape[:-2]
    batches = [()] if not batch_shape else [tuple(0 for _ in batch_shape), tuple(d - 1 for d in batch_shape)]
    rows = _pick(M, [M // 2, M - 2], rng)
    cols = _pick(N, [N // 2, N - 2, inf["tail_col"]], rng)
    for bidx in batches:
        # broadcast: a size-1 batch dimension of an operand reads matrix 0
        pa_idx = tuple(0 if d == 1 else i for d, i in zip(sa[:-2], bidx[len(bidx) - len(sa[:-2]):]))
        pb_idx = tuple(0 if d == 1 else i for d, i in zip(sb[:-2], bidx[len(bidx) - len(sb[:-2]):]))
        a_sub = _rows(pa, sa, pa_idx, rows)
        b_sub = _cols(pb, sb, pb_idx, cols)
        o = oracle.matmul_at(a_sub, b_sub, dt, np.arange(rows.size * cols.size))
        yb = Y[bidx] if bidx else Y
        ys = yb[torch.from_numpy(rows).to(dev)][:, torch.from_numpy(cols).to(dev)]
        rep = check(synth.from_torch(ys), o, dt, K, 1.0, 1.0, exact=True)
        assert rep.ok, f"{sa} x {sb} batch {bidx}: {rep}"
    del Y
    torch.cuda.empty_cache()


def test_matmul_integer_beyond_4gib(dev):
    """MatMulInteger (UINT8 x INT8, no zero points) on the tiled INT8 kernel
    with a 4.6 GB B; INT32 results modulo 2^32 are compared exactly."""
    sa, sb = (64, 65536), (65536, 70000)
    assert sb[0] * sb[1] > FOUR_GIB
    plan = mm.IntPlan(sa, sb, mm.UINT8, mm.INT8)
    assert mm.ALGO_NAMES[plan.algo] == "general", plan.info()
    pa, pb = _pattern(None, [78, 0], signed=False), _pattern(None, [78, 1], signed=True)
    A = _device(pa, None, sa, dev)
    B = _device(pb, None, sb, dev)
    Y = torch.full(plan.output_shape, 0x5EADBEEF, dtype=torch.int32, device=dev)
    plan.execute(A, B, Y)
    torch.cuda.synchronize()
    del A, B
    rng = np.random.default_rng(6)
    rows = _pick(sa[0], [], rng)
    cols = _pick(sb[1], [sb[1] // 2], rng)
    a_sub = _rows(pa, sa, (), rows)
    b_sub = _cols(pb, sb, (), cols)
    o = oracle.matmul_integer_at(a_sub, b_sub, np.arange(rows.size * cols.size)).reshape(rows.size, cols.size)
    ys = Y[torch.from_numpy(rows).to(dev)][:, torch.from_numpy(cols).to(dev)].cpu().numpy()
    assert np.array_equal(ys, o)
    del Y
    torch.cuda.empty_cache()
