"""HIP graph capture of mm_execute and mm_execute_noalloc.

No execution path allocates, synchronises or issues a hipMemsetAsync at
execute time (workspaces come from plan creation, zero outputs from a fill
kernel), so the calls can be captured.  Each case captures one call,
replays the graph several times with the program's own eager work and a
synchronisation between replays, and checks every replay bit for bit
against an eager execution.
"""
import pytest

from onnx_broadcast_matmul_amd import binding as mm
from onnx_broadcast_matmul_amd import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

U1 = ("uniform", -1.0, 1.0)

# (A shape, B shape, element type, forced algorithm or 0, the algorithm the plan must run)
CASES = [
    ((4, 32, 512, 128), (4, 32, 128, 512), mm.BFLOAT16, 0, "general"),  # persistent tiles
    ((16, 512, 256), (256, 1000), mm.FLOAT16, 0, "general"),            # one-tile kernel, ragged N
    ((64, 16384), (16384, 64), mm.FLOAT, 0, "split_k"),                 # workspace partials + reduction
    ((1, 4096), (4096, 8704), mm.FLOAT, 0, "skinny_m"),                 # skinny-M with K cut
    ((8192, 1024), (1024, 8), mm.FLOAT16, 0, "skinny_n"),
    ((4, 64, 96), (96, 80), mm.FLOAT, 0, "direct"),
    ((3, 4, 0), (0, 5), mm.FLOAT, 0, "zero_fill"),                       # K = 0: the fill kernel
]


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    mm.lib()
    return torch.device("cuda:0")


def _operand(shape, dt, seed, dev):
    if 0 in shape:
        return torch.empty(shape, dtype=mm.torch_dtype(dt), device=dev)
    return synth.as_torch(synth.generate(shape, dt, U1, seed), dt).to(dev)


@pytest.mark.parametrize("noalloc", [False, True], ids=["execute", "noalloc"])
@pytest.mark.parametrize("sa,sb,dt,algo,want", CASES, ids=lambda v: "x".join(map(str, v)) if isinstance(v, tuple) else None)
def test_graph_replay_matches_eager(sa, sb, dt, algo, want, noalloc, dev):
    plan = mm.Plan(sa, sb, dt, force_algo=algo)
    assert mm.ALGO_NAMES[plan.algo] == want
    if sa == (4, 32, 512, 128):
        assert plan.info()["tile"] == 11  # the persistent kernel
    run = plan.execute_noalloc if noalloc else plan.execute
    A = _operand(sa, dt, [93, 0], dev)
    B = _operand(sb, dt, [93, 1], dev)
    tdt = mm.torch_dtype(dt)
    ref = torch.full(plan.output_shape, float("nan"), dtype=tdt, device=dev)
    run(A, B, ref)
    torch.cuda.synchronize()

    Y = torch.full(plan.output_shape, float("nan"), dtype=tdt, device=dev)
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()  # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(graph, stream=side):
        run(A, B, Y)
    torch.cuda.synchronize()
    for replay in range(4):
        Y.fill_(float("nan"))  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(Y.view(torch.uint8), ref.view(torch.uint8)), f"replay {replay} differs from eager execution"
