"""GPU parity of the narrowing epilogue at its edges, bit for bit.

The final narrowing (page "MatMul Kernel Design", section "Types and
algorithm selection": FP32 accumulation, one narrowing at the end; read as
round to nearest even with IEEE overflow and FP16 subnormals kept) must
give, for every algorithm, exactly the oracle value rounded once to the
output type -- including outputs past the type's largest finite value
(+-Inf), outputs in the FP16 subnormal range and outputs exactly halfway
between two representable values.

Inputs are integers times a power of two per row of A and per column of B
(``synth.generate_scaled_int``): every product is exact in FP32 and every
partial sum is an integer below 2^24 times the output's common power of
two, so the FP32 accumulator holds the exact sum whatever the summation
order, and both sides then narrow the same exact value.  The overflow cases
of BF16 and FP32 use non-negative integers, so no partial sum can overflow
where the full sum does not.
"""
import numpy as np
import pytest

import oracle
from oracle.compare import abs_max, check
from onnx_broadcast_matmul_amd import binding as mm
from onnx_broadcast_matmul_amd import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

DT_IDS = {mm.FLOAT: "fp32", mm.FLOAT16: "fp16", mm.BFLOAT16: "bf16"}

# (element type, integer range, exponent range, what the outputs reach)
EDGE_CASES = [
    pytest.param(mm.FLOAT16, (-31, 31), (-14, 7), id="fp16-overflow-subnormal-ties"),
    pytest.param(mm.BFLOAT16, (-31, 31), (-20, 20), id="bf16-ties"),
    pytest.param(mm.BFLOAT16, (0, 31), (40, 60), id="bf16-overflow"),
    pytest.param(mm.FLOAT, (0, 31), (40, 60), id="fp32-overflow"),
]

# Shapes per forced algorithm: (A shape, B shape, split count).  Skinny-M
# covers the packed-dot kernel (rows of 16-byte chunks) with and without a
# K split and the element-wise one; skinny-N the eight-column matrix-core
# kernel and the general one.
ALGO_SHAPES = {
    mm.ALGO_DIRECT: [((2, 40, 96), (96, 70), 0)],
    mm.ALGO_GENERAL: [((2, 100, 200), (200, 150), 0), ((300, 256), (256, 264), 0)],
    mm.ALGO_SPLIT_K: [((64, 2048), (2048, 48), 4), ((37, 1000), (1000, 29), 3)],
    mm.ALGO_SKINNY_M: [((3, 2048), (2048, 256), 0), ((1, 2048), (2048, 256), 4), ((5, 777), (777, 99), 2)],
    mm.ALGO_SKINNY_N: [((500, 1024), (1024, 8), 0), ((300, 520), (520, 5), 0)],
}


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    mm.lib()
    return torch.device("cuda:0")


def _edge_counts(o: np.ndarray, dt: int):
    """How many oracle values overflow, are FP16 subnormal, or are ties."""
    ref = oracle.narrow(o, dt)
    if dt == mm.FLOAT:
        return {"overflow": int(np.isinf(ref).sum())}
    rv = oracle.decode(ref, dt)
    p, emin = (11, -14) if dt == mm.FLOAT16 else (8, -126)
    ax = np.abs(o)
    fin = np.isfinite(rv) & (ax > 0)
    e = np.floor(np.log2(np.where(fin, ax, 1.0)))
    ulp = np.ldexp(1.0, (np.maximum(e, emin) - (p - 1)).astype(np.int64))
    q = np.where(fin, ax / ulp, 0.0)
    return {
        "overflow": int(np.isinf(rv).sum()),
        "subnormal": int((fin & (np.abs(rv) < 2.0 ** emin) & (rv != 0)).sum()),
        "tie": int((fin & (q - np.floor(q) == 0.5)).sum()),
    }


@pytest.mark.parametrize("algo", list(ALGO_SHAPES), ids=lambda a: mm.ALGO_NAMES[a])
@pytest.mark.parametrize("dt,ints,exps", EDGE_CASES)
def test_narrowing_edges_bit_exact(dt, ints, exps, algo, dev):
    totals = {}
    for i, (sa, sb, split) in enumerate(ALGO_SHAPES[algo]):
        print(f"\n[narrowing] {DT_IDS[dt]} {mm.ALGO_NAMES[algo]} {sa} x {sb} split={split}", flush=True)
        a = synth.generate_scaled_int(sa, dt, [90, algo, i, 0], ints, exps, "a")
        b = synth.generate_scaled_int(sb, dt, [90, algo, i, 1], ints, exps, "b")
        plan = mm.Plan(sa, sb, dt, force_algo=algo, split_k=split)
        assert plan.algo == algo
        A = synth.as_torch(a, dt).to(dev)
        B = synth.as_torch(b, dt).to(dev)
        Y = torch.full(plan.output_shape, float("nan"), dtype=mm.torch_dtype(dt), device=dev)
        plan.execute(A, B, Y)
        torch.cuda.synchronize()
        o = oracle.matmul(a, b, dt)
        rep = check(synth.from_torch(Y), o, dt, sa[-1], abs_max(a, dt), abs_max(b, dt), exact=True)
        assert rep.ok, f"{sa} x {sb} {DT_IDS[dt]} {mm.ALGO_NAMES[algo]} split={plan.info()['split_k']}: {rep}"
        for k, v in _edge_counts(o, dt).items():
            totals[k] = totals.get(k, 0) + v
    # the inputs must actually reach the edges this case is about
    if dt == mm.FLOAT16:
        assert totals["overflow"] > 0 and totals["subnormal"] > 0 and totals["tie"] > 0, totals
    elif ints[0] < 0:
        assert totals["tie"] > 0, totals
    else:
        assert totals["overflow"] > 0, totals
