"""mm_execute_noalloc (the entry point for callers that cannot allocate
device memory) against mm_execute, through the C ABI.

Both run the same plan with the same kernels; only where the split partial
sums live differs (the library's fixed per-device array instead of the
plan's workspace), so the outputs must be equal bit for bit, and both must
meet the oracle's tolerance.  Each case makes two no-allocation calls in a
row, the second on a smaller product, then repeats the first (the array
then holds the smaller call's stale partial sums), and checks every output.
"""
import numpy as np
import pytest

import oracle
from oracle.compare import abs_max, check
from onnx_broadcast_matmul_amd import binding as mm
from onnx_broadcast_matmul_amd import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

U1 = ("uniform", -1.0, 1.0)

# (larger product, smaller product), element type, forced algorithm, split count
CASES = [
    pytest.param(((64, 65536), (65536, 64)), ((48, 16384), (16384, 40)), mm.FLOAT, mm.ALGO_SPLIT_K, 0,
                 id="fp32-split-k"),
    pytest.param(((256, 4096), (4096, 512)), ((100, 2048), (2048, 130)), mm.FLOAT16, mm.ALGO_SPLIT_K, 8,
                 id="fp16-split-k"),
    pytest.param(((3, 1, 8192), (3, 8192, 1032)), ((2, 1, 4096), (2, 4096, 264)), mm.BFLOAT16, mm.ALGO_SKINNY_M, 16,
                 id="bf16-skinny-m-split"),
    pytest.param(((64, 8192), (8192, 48)), ((20, 2048), (2048, 16)), mm.DOUBLE, mm.ALGO_SPLIT_K, 0,
                 id="fp64-split-k"),
    pytest.param(((2, 100, 300), (300, 200)), ((50, 64), (64, 30)), mm.FLOAT, mm.ALGO_GENERAL, 0,
                 id="fp32-general-no-workspace"),
]


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    mm.lib()
    return torch.device("cuda:0")


def _sentinel(shape, dt, dev):
    return torch.full(shape, float("nan"), dtype=mm.torch_dtype(dt), device=dev)


@pytest.mark.parametrize("big,small,dt,algo,split", CASES)
def test_noalloc_equals_execute(big, small, dt, algo, split, dev):
    runs = []
    for i, (sa, sb) in enumerate((big, small)):
        plan = mm.Plan(sa, sb, dt, force_algo=algo, split_k=split)
        assert plan.algo == algo
        if algo != mm.ALGO_GENERAL:
            assert 0 < plan.workspace_bytes <= 16 << 20, plan.workspace_bytes
        a = synth.generate(sa, dt, U1, [95, i, 0])
        b = synth.generate(sb, dt, U1, [95, i, 1])
        A, B = synth.as_torch(a, dt).to(dev), synth.as_torch(b, dt).to(dev)
        ref = _sentinel(plan.output_shape, dt, dev)
        plan.execute(A, B, ref)
        runs.append((plan, a, b, A, B, ref))
    torch.cuda.synchronize()
    print(f"\n[noalloc] {mm.ALGO_NAMES[algo]} {big} then {small}", flush=True)
    # two no-allocation calls in a row, the second smaller, then the first again
    outs = []
    for plan, a, b, A, B, ref in runs + runs[:1]:
        y = _sentinel(plan.output_shape, dt, dev)
        plan.execute_noalloc(A, B, y)
        outs.append(y)
    torch.cuda.synchronize()
    for (plan, a, b, A, B, ref), y in zip(runs + runs[:1], outs):
        yr, yn = synth.from_torch(ref), synth.from_torch(y)
        assert np.array_equal(yr.view(np.uint8), yn.view(np.uint8)), f"{plan.a_shape} x {plan.b_shape}"
        rep = check(yn, oracle.matmul(a, b, dt), dt, plan.a_shape[-1], abs_max(a, dt), abs_max(b, dt))
        assert rep.ok, f"{plan.a_shape} x {plan.b_shape}: {rep}"


def test_noalloc_rejects_large_workspace_and_other_plans(dev):
    """A plan needing more than the 16 MiB array is refused before any
    launch (the output keeps its sentinel); Gemm plans run elsewhere."""
    sa, sb = (512, 8192), (8192, 512)
    plan = mm.Plan(sa, sb, mm.FLOAT, force_algo=mm.ALGO_SPLIT_K, split_k=32)
    assert plan.workspace_bytes > 16 << 20
    A = torch.zeros(sa, dtype=torch.float32, device=dev)
    B = torch.zeros(sb, dtype=torch.float32, device=dev)
    Y = _sentinel(plan.output_shape, mm.FLOAT, dev)
    with pytest.raises(mm.MMError) as ei:
        plan.execute_noalloc(A, B, Y)
    assert ei.value.status == mm.ERR_TOO_LARGE and "16777216" in str(ei.value)
    torch.cuda.synchronize()
    assert torch.isnan(Y).all().item()
    g = mm.GemmPlan((64, 128), (128, 32), mm.FLOAT)
    lib = mm.lib()
    st = lib.mm_execute_noalloc(g.handle, None, None, None, None)
    assert st == mm.ERR_BAD_OPTION
