"""GPU parity: the HIP kernels behind the C ABI against the fp64 CPU oracle.

Tolerances (oracle/compare.py): FP32 max|y-o| <= 1e-4*sqrt(K)*max|A|*max|B|;
FP16/BF16 within 2 ulp of the narrowed oracle value (or the FP32 rule for
results near zero); DOUBLE max|y-o| <= 2*gamma_K*K*max|A|*max|B| (both sides
round their products); bit-exact on small-integer-valued inputs.  DOUBLE has
no skinny kernels, so its cases skip the forced skinny algorithms.  Every
algorithm is forced on every element type over shapes that span several
tiles and ragged tails, plus broadcast, rank-one, empty, K == 0, unaligned
and special-value cases, and the full-size workload products on every
output.
"""
import numpy as np
import pytest

import oracle
from oracle.compare import abs_max, check, gemm_tolerance
from onnx_broadcast_matmul_amd import binding as mm
from onnx_broadcast_matmul_amd import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

DTYPES = [mm.FLOAT, mm.FLOAT16, mm.BFLOAT16, mm.DOUBLE]
DT_IDS = {mm.FLOAT: "fp32", mm.FLOAT16: "fp16", mm.BFLOAT16: "bf16", mm.DOUBLE: "fp64"}
ALGOS = [mm.ALGO_DIRECT, mm.ALGO_SKINNY_M, mm.ALGO_SKINNY_N, mm.ALGO_SPLIT_K, mm.ALGO_GENERAL]
U1 = ("uniform", -1.0, 1.0)


def algos_for(dt, algos=ALGOS):
    """The forcible algorithms of an element type (DOUBLE has no skinny kernels)."""
    if dt == mm.DOUBLE:
        return [a for a in algos if a not in (mm.ALGO_SKINNY_M, mm.ALGO_SKINNY_N)]
    return list(algos)


def dt_algo_params(algos=ALGOS):
    return [pytest.param(dt, a, id=f"{mm.ALGO_NAMES[a]}-{DT_IDS[dt]}") for dt in DTYPES for a in algos_for(dt, algos)]


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    mm.lib()  # the native library must load: no fallback exists
    return torch.device("cuda:0")


def _sentinel(shape, dt, dev):
    # NaN everywhere, so an output the kernels never write fails the check
    return torch.full(shape, float("nan"), dtype=mm.torch_dtype(dt), device=dev)


def run_plan(plan, a, b, dt, dev):
    A = synth.as_torch(a, dt).to(dev)
    B = synth.as_torch(b, dt).to(dev)
    Y = _sentinel(plan.output_shape, dt, dev)
    plan.execute(A, B, Y)
    torch.cuda.synchronize()
    return Y


def parity(sa, sb, dt, dev, algo=0, tile=0, split=0, dist=U1, seed=0, exact=False):
    a = synth.generate(sa, dt, dist, [seed, 0])
    b = synth.generate(sb, dt, dist, [seed, 1])
    plan = mm.Plan(sa, sb, dt, force_algo=algo, tile=tile, split_k=split)
    if algo:
        assert plan.algo == algo
    Y = run_plan(plan, a, b, dt, dev)
    o = oracle.matmul(a, b, dt)
    assert tuple(Y.shape) == o.shape
    rep = check(synth.from_torch(Y), o, dt, sa[-1], abs_max(a, dt), abs_max(b, dt), exact=exact)
    assert rep.ok, f"{sa} x {sb} {DT_IDS[dt]} algo={mm.ALGO_NAMES[plan.algo]} tile={plan.info()['tile']}: {rep}"
    return plan, Y, rep


RAGGED = [
    ((300, 520), (520, 200)),          # several tiles, ragged M/N tails, 16-byte rows
    ((67, 77), (77, 19)),              # odd sizes: element-wise loads
    ((2, 3, 33, 40), (40, 24)),        # batch folded into M (B shared)
    ((3, 1, 17, 64), (2, 64, 48)),     # both operands broadcast
    ((5, 130), (130, 3)),              # tiny N
    ((2, 1, 1000), (2, 1000, 72)),     # M == 1 per batch, K tail vs 64-wide stages
]


@pytest.mark.parametrize("dt,algo", dt_algo_params())
@pytest.mark.parametrize("sa,sb", RAGGED, ids=lambda s: "x".join(map(str, s)))
def test_forced_algorithms(sa, sb, dt, algo, dev):
    parity(sa, sb, dt, dev, algo=algo)


@pytest.mark.parametrize("dt", DTYPES, ids=DT_IDS.get)
def test_every_tile(dt, dev):
    for t in range(1, len(mm.tile_configs(dt)) + 1):
        parity((300, 520), (520, 200), dt, dev, algo=mm.ALGO_GENERAL, tile=t, seed=t)
        parity((2, 1, 96, 1000), (3, 1000, 72), dt, dev, algo=mm.ALGO_GENERAL, tile=t, seed=t)
        parity((3, 250, 770), (770, 130), dt, dev, algo=mm.ALGO_SPLIT_K, tile=t, split=5, seed=t)


@pytest.mark.parametrize("dt", DTYPES, ids=DT_IDS.get)
@pytest.mark.parametrize("split", [2, 3, 7, 16, 33, 64, 100, 300])
def test_split_counts(dt, split, dev):
    """Every partition-lane width of the split-K reduction, with output
    counts that are (64 x 40) and are not (37 x 29) a multiple of four;
    small-integer inputs must stay bit-exact whatever the split."""
    for sa, sb in [((64, 19200), (19200, 40)), ((37, 19200), (19200, 29))]:
        plan, _, _ = parity(sa, sb, dt, dev, algo=mm.ALGO_SPLIT_K, split=split, seed=split)
        # the plan rounds partitions to whole LDS stages, so the count may shrink a little
        assert split // 2 < plan.info()["split_k"] <= split
        parity(sa, sb, dt, dev, algo=mm.ALGO_SPLIT_K, split=split, seed=split, dist=("int",), exact=True)


@pytest.mark.parametrize("dt", [mm.FLOAT, mm.FLOAT16, mm.BFLOAT16], ids=DT_IDS.get)
@pytest.mark.parametrize("split", [64, 100])
def test_gemm_split_reduction_epilogue(dt, split, dev):
    """The reduction over more partitions than partition lanes (each lane
    then adds several partitions in order) applies the Gemm epilogue (alpha,
    beta, per-column and full C) when it writes each output."""
    M, N, K = 64, 40, 19200
    for i, layout in enumerate([("N",), ("M", "N")]):
        cs = _cs(layout, M, N)
        a = synth.generate((M, K), dt, U1, [80 + i, 0])
        b = synth.generate((N, K), dt, U1, [80 + i, 1])
        c = synth.generate(cs, dt, U1, [80 + i, 2])
        plan = mm.GemmPlan((M, K), (N, K), dt, False, True, cs, 0.5, -2.0, force_algo=mm.ALGO_SPLIT_K, split_k=split)
        assert plan.info()["split_k"] > 32
        Y = _sentinel((M, N), dt, dev)
        plan.execute(synth.as_torch(a, dt).to(dev), synth.as_torch(b, dt).to(dev), Y, synth.as_torch(c, dt).to(dev))
        torch.cuda.synchronize()
        o = oracle.gemm(a, b, dt, False, True, c, 0.5, -2.0)
        tol = gemm_tolerance(K, abs_max(a, dt), abs_max(b, dt), abs_max(c, dt), 0.5, -2.0)
        rep = check(synth.from_torch(Y), o, dt, K, abs_max(a, dt), abs_max(b, dt), tol=tol)
        assert rep.ok, f"split {split} C={cs} {DT_IDS[dt]}: {rep}"


@pytest.mark.parametrize("dt", [mm.FLOAT, mm.FLOAT16, mm.BFLOAT16], ids=DT_IDS.get)
@pytest.mark.parametrize("split", [1, 2, 3, 7, 16, 64])
def test_skinny_m_split_counts(dt, split, dev):
    """Skinny-M with K cut into chunks over workgroups: a K that is not a
    multiple of the 64-row chunk unit, a folded batch (rows in two row
    groups), broadcast batches, unaligned columns (element-wise loads), and
    small-integer exactness whatever the chunk count."""
    # The last two have K and N multiples of 8 (rows of 16-byte chunks): for
    # the 16-bit types they run the packed-dot kernel's 2-row and 8-row
    # instances.
    cases = [((1, 4100), (4100, 300)), ((5, 2, 3, 1000), (1000, 520)),
             ((3, 1, 4, 640), (2, 640, 136)), ((2, 1111), (1111, 77)),
             ((2, 4096), (4096, 264)), ((6, 2048), (2048, 136))]
    for i, (sa, sb) in enumerate(cases):
        plan, _, _ = parity(sa, sb, dt, dev, algo=mm.ALGO_SKINNY_M, split=split, seed=60 + i)
        assert 1 <= plan.info()["split_k"] <= split
        parity(sa, sb, dt, dev, algo=mm.ALGO_SKINNY_M, split=split, seed=60 + i, dist=("int",), exact=True)


@pytest.mark.parametrize("dt", [mm.FLOAT, mm.FLOAT16, mm.BFLOAT16], ids=DT_IDS.get)
def test_skinny_n_eight_columns(dt, dev):
    """Eight output columns: ragged row counts, K from one chunk to the
    4096 limit of the register-slice kernel and past it, batched and
    broadcast B, and small-integer exactness."""
    cases = [((37, 8), (8, 8)), ((1000, 520), (520, 8)), ((300, 4096), (4096, 8)),
             ((3, 50, 1024), (3, 1024, 8)), ((2, 40, 2048), (2048, 8)), ((70, 4104), (4104, 8))]
    for i, (sa, sb) in enumerate(cases):
        plan, _, _ = parity(sa, sb, dt, dev, algo=mm.ALGO_SKINNY_N, seed=40 + i)
        parity(sa, sb, dt, dev, algo=mm.ALGO_SKINNY_N, seed=40 + i, dist=("int",), exact=True)


@pytest.mark.parametrize("dt,algo", dt_algo_params())
def test_small_integer_bit_exact(dt, algo, dev):
    parity((2, 130, 1000), (1000, 70), dt, dev, algo=algo, dist=("int",), exact=True)
    parity((70, 333), (333, 9), dt, dev, algo=algo, dist=("int",), exact=True)


@pytest.mark.parametrize("dt,algo", dt_algo_params([0] + ALGOS))
def test_broadcast_equals_materialized(dt, algo, dev):
    """Zero-stride broadcast reads give bitwise the same result as an
    explicitly repeated batch under the same kernel."""
    sa, sb = (3, 1, 64, 96), (1, 4, 96, 80)
    a = synth.generate(sa, dt, U1, [7, 0])
    b = synth.generate(sb, dt, U1, [7, 1])
    ar = np.ascontiguousarray(np.broadcast_to(a, (3, 4, 64, 96)))
    br = np.ascontiguousarray(np.broadcast_to(b, (3, 4, 96, 80)))
    p1 = mm.Plan(sa, sb, dt, force_algo=algo)
    p2 = mm.Plan(ar.shape, br.shape, dt, force_algo=p1.algo, tile=p1.info()["tile"])
    y1 = synth.from_torch(run_plan(p1, a, b, dt, dev))
    y2 = synth.from_torch(run_plan(p2, ar, br, dt, dev))
    assert np.array_equal(y1.view(np.uint8), y2.view(np.uint8))


@pytest.mark.parametrize("dt", DTYPES, ids=DT_IDS.get)
def test_rank_one(dt, dev):
    K = 96
    _, yv, _ = parity((K,), (K, 80), dt, dev)
    assert tuple(yv.shape) == (80,)
    _, ym, _ = parity((4, 64, K), (K,), dt, dev)
    assert tuple(ym.shape) == (4, 64)
    _, ys, _ = parity((K,), (K,), dt, dev)
    assert tuple(ys.shape) == ()
    _, yb, _ = parity((K,), (3, K, 40), dt, dev)
    assert tuple(yb.shape) == (3, 40)
    for algo in algos_for(dt):
        a = synth.generate((K,), dt, U1, [3, 0])
        b = synth.generate((K, 80), dt, U1, [3, 1])
        y1 = synth.from_torch(run_plan(mm.Plan((K,), (K, 80), dt, force_algo=algo), a, b, dt, dev))
        y2 = synth.from_torch(run_plan(mm.Plan((1, K), (K, 80), dt, force_algo=algo), a[None, :], b, dt, dev))
        assert np.array_equal(y1.view(np.uint8), y2.reshape(-1).view(np.uint8))


@pytest.mark.parametrize("dt", DTYPES, ids=DT_IDS.get)
def test_empty_and_zero_k(dt, dev):
    for sa, sb in [((3, 0, 5), (5, 4)), ((0, 4, 5), (1, 5, 6)), ((4, 5), (5, 0))]:
        plan = mm.Plan(sa, sb, dt)
        assert plan.algo == mm.ALGO_EMPTY and plan.output_numel == 0
        plan.execute_ptr(0, 0, 0)  # launches nothing, reads nothing
    for sa, sb in [((3, 4, 0), (0, 5)), ((0,), (0, 7)), ((2, 1, 6, 0), (3, 0, 2))]:
        plan = mm.Plan(sa, sb, dt)
        assert plan.algo == mm.ALGO_ZERO_FILL
        Y = _sentinel(plan.output_shape, dt, dev)
        plan.execute_ptr(0, 0, Y.data_ptr(), torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        assert torch.all(Y == 0).item()


@pytest.mark.parametrize("dt,algo", dt_algo_params())
def test_deterministic(dt, algo, dev):
    sa, sb = (2, 200, 700), (700, 150)
    a = synth.generate(sa, dt, U1, [11, 0])
    b = synth.generate(sb, dt, U1, [11, 1])
    plan = mm.Plan(sa, sb, dt, force_algo=algo)
    y1 = synth.from_torch(run_plan(plan, a, b, dt, dev))
    y2 = synth.from_torch(run_plan(plan, a, b, dt, dev))
    assert np.array_equal(y1.view(np.uint8), y2.view(np.uint8))


@pytest.mark.parametrize("dt,algo", dt_algo_params())
def test_unaligned_pointers(dt, algo, dev):
    """Operands that start one element past a 16-byte boundary take the
    element-wise load paths."""
    sa, sb = (96, 256), (256, 64)
    a = synth.generate(sa, dt, U1, [13, 0])
    b = synth.generate(sb, dt, U1, [13, 1])
    plan = mm.Plan(sa, sb, dt, force_algo=algo)
    A = torch.empty(a.size + 1, dtype=mm.torch_dtype(dt), device=dev)[1:].view(sa)
    B = torch.empty(b.size + 1, dtype=mm.torch_dtype(dt), device=dev)[1:].view(sb)
    A.copy_(synth.as_torch(a, dt).to(dev))
    B.copy_(synth.as_torch(b, dt).to(dev))
    Yb = torch.full((96 * 64 + 1,), float("nan"), dtype=mm.torch_dtype(dt), device=dev)
    Y = Yb[1:].view(96, 64)
    plan.execute(A, B, Y)
    torch.cuda.synchronize()
    rep = check(synth.from_torch(Y), oracle.matmul(a, b, dt), dt, 256, abs_max(a, dt), abs_max(b, dt))
    assert rep.ok, str(rep)


@pytest.mark.parametrize("dt,algo", dt_algo_params())
def test_special_values(dt, algo, dev):
    """An infinity or NaN in A reaches exactly the outputs of its row, as in
    the oracle (NaN stays NaN through the narrowing)."""
    sa, sb = (40, 128), (128, 24)
    a = synth.generate(sa, dt, U1, [17, 0])
    b = synth.generate(sb, dt, U1, [17, 1])
    inf_bits = {mm.FLOAT: np.float32(np.inf), mm.FLOAT16: np.uint16(0x7C00), mm.BFLOAT16: np.uint16(0x7F80),
                mm.DOUBLE: np.float64(np.inf)}[dt]
    nan_bits = {mm.FLOAT: np.float32(np.nan), mm.FLOAT16: np.uint16(0x7E00), mm.BFLOAT16: np.uint16(0x7FC0),
                mm.DOUBLE: np.float64(np.nan)}[dt]
    a[3, 5] = inf_bits
    a[7, 9] = nan_bits
    plan = mm.Plan(sa, sb, dt, force_algo=algo)
    Y = run_plan(plan, a, b, dt, dev)
    o = oracle.matmul(a, b, dt)
    av = np.asarray(a, dtype=np.float64) if dt in (mm.FLOAT, mm.DOUBLE) else oracle.decode(a, dt)
    finite = np.isfinite(av)
    rep = check(synth.from_torch(Y), o, dt, 128, float(np.abs(av[finite]).max()), abs_max(b, dt))
    assert rep.ok, str(rep)


@pytest.mark.parametrize("dt", [mm.FLOAT16, mm.BFLOAT16], ids=DT_IDS.get)
@pytest.mark.parametrize("m,n", [(8192, 11000), (8192, 11002), (2048, 11000), (2048, 9000)])
def test_tail_split(dt, m, n, dev):
    """Last-round balancing: columns [0, tail_col) run with the plan's tile
    and the rest with the tail tile.  The result equals, bit for bit, each
    column range of a single launch forced to the corresponding tile (a
    tile's per-element summation order does not depend on N), and matches
    the oracle on sampled outputs around the boundary.  N = 11002 has rows
    that are not whole 16-byte chunks (element-wise loads and stores); the
    2048-row products take three-stage tail tiles (256 x 128, 128 x 64)."""
    sa, sb = (m, 128), (128, n)
    a = synth.generate(sa, dt, ("int",), [31, 0])
    b = synth.generate(sb, dt, ("int",), [31, 1])
    plan = mm.Plan(sa, sb, dt)
    inf = plan.info()
    assert plan.algo == mm.ALGO_GENERAL and inf["tail_col"] > 0, inf
    c = inf["tail_col"]
    y = synth.from_torch(run_plan(plan, a, b, dt, dev))
    ym = synth.from_torch(run_plan(mm.Plan(sa, sb, dt, force_algo=mm.ALGO_GENERAL, tile=inf["tile"]), a, b, dt, dev))
    yr = synth.from_torch(run_plan(mm.Plan(sa, sb, dt, force_algo=mm.ALGO_GENERAL, tile=inf["tail_tile"]), a, b, dt, dev))
    assert np.array_equal(y[:, :c], ym[:, :c])
    assert np.array_equal(y[:, c:], yr[:, c:])
    rng = np.random.default_rng(3)
    rows = rng.integers(0, sa[0], 400)
    cols = np.concatenate([rng.integers(0, n, 200), rng.integers(c - 8, min(n, c + 8), 200)])
    idx = np.unique(rows * n + cols)
    o = oracle.matmul_at(a, b, dt, idx)
    rep = check(y.reshape(-1)[idx], o, dt, sa[-1], abs_max(a, dt), abs_max(b, dt), exact=True)
    assert rep.ok, str(rep)


@pytest.mark.parametrize("dt,algo", dt_algo_params([0] + ALGOS))
def test_constant_b(dt, algo, dev):
    """A plan-owned constant B: after the copy the source buffer is
    overwritten and freed, and mm_execute_constant_b still equals
    mm_execute with the original B bit for bit; setting B again replaces it.
    B is broadcast over A's batch (kept dense by a second batch axis)."""
    sa, sb = (3, 2, 70, 300), (2, 300, 90)
    a = synth.generate(sa, dt, U1, [41, 0])
    b1 = synth.generate(sb, dt, U1, [41, 1])
    b2 = synth.generate(sb, dt, U1, [41, 2])
    plan = mm.Plan(sa, sb, dt, force_algo=algo)
    A = synth.as_torch(a, dt).to(dev)
    src = synth.as_torch(b1, dt).to(dev)
    plan.set_constant_b(src)
    assert plan.has_constant_b
    src.fill_(float("nan"))
    del src
    torch.cuda.synchronize()
    for b in (b1, b2):
        if b is b2:
            plan.set_constant_b(synth.as_torch(b2, dt).to(dev))
        Yc = _sentinel(plan.output_shape, dt, dev)
        plan.execute_constant_b(A, Yc)
        Ye = run_plan(plan, a, b, dt, dev)
        torch.cuda.synchronize()
        assert np.array_equal(synth.from_torch(Yc).view(np.uint8), synth.from_torch(Ye).view(np.uint8))
        rep = check(synth.from_torch(Yc), oracle.matmul(a, b, dt), dt, sa[-1], abs_max(a, dt), abs_max(b, dt))
        assert rep.ok, str(rep)


@pytest.mark.parametrize("dt", [mm.FLOAT16, mm.BFLOAT16], ids=DT_IDS.get)
def test_constant_b_prepacked(dt, dev):
    """A 16-bit GENERAL plan keeps its constant B also prepacked in the tiled
    kernel's stage order; for every tile of the table, over two B matrices,
    ragged M, N (a multiple of 8) and a K that leaves the last stage partly
    filled, mm_execute_constant_b equals mm_execute with the same B bit for
    bit, and stays so after B is replaced."""
    sa, sb = (2, 3, 70, 520), (2, 1, 520, 200)
    a = synth.generate(sa, dt, U1, [45, 0])
    b1 = synth.generate(sb, dt, U1, [45, 1])
    b2 = synth.generate(sb, dt, U1, [45, 2])
    A = synth.as_torch(a, dt).to(dev)
    cfgs = mm.tile_configs(dt)
    for t in range(1, len(cfgs) + 1):
        plan = mm.Plan(sa, sb, dt, force_algo=mm.ALGO_GENERAL, tile=t)
        for b in (b1, b2):
            plan.set_constant_b(synth.as_torch(b, dt).to(dev))
            # prepacked for the tiles that stage 64 elements of K
            assert plan.info()["constant_b_packed"] == (1 if cfgs[t - 1][2] == 64 else 0)
            Yc = _sentinel(plan.output_shape, dt, dev)
            plan.execute_constant_b(A, Yc)
            Ye = run_plan(plan, a, b, dt, dev)
            torch.cuda.synchronize()
            assert np.array_equal(synth.from_torch(Yc), synth.from_torch(Ye)), f"tile {t}"
        rep = check(synth.from_torch(Yc), oracle.matmul(a, b2, dt), dt, sa[-1], abs_max(a, dt), abs_max(b2, dt))
        assert rep.ok, f"tile {t}: {rep}"
    # not prepacked: N not a multiple of 8, and a non-GENERAL algorithm
    p2 = mm.Plan((70, 520), (520, 90), dt, force_algo=mm.ALGO_GENERAL)
    p2.set_constant_b(synth.as_torch(synth.generate((520, 90), dt, U1, [45, 3]), dt).to(dev))
    assert p2.info()["constant_b_packed"] == 0
    p3 = mm.Plan((70, 520), (520, 96), dt, force_algo=mm.ALGO_SPLIT_K)
    p3.set_constant_b(synth.as_torch(synth.generate((520, 96), dt, U1, [45, 4]), dt).to(dev))
    assert p3.info()["constant_b_packed"] == 0


@pytest.mark.parametrize("dt", [mm.FLOAT16, mm.BFLOAT16], ids=DT_IDS.get)
@pytest.mark.parametrize("sa,sb", [
    ((16, 1024, 128), (16, 128, 2048)),  # 512 tiles: two per workgroup
    ((1024, 64), (64, 1024)),            # one stage per tile
    ((4, 512, 192), (192, 768)),         # broadcast B, three stages per tile
    ((2, 3, 512, 256), (3, 256, 512)),   # broadcast A batch dimension
], ids=lambda s: "x".join(map(str, s)))
def test_persistent_tile(sa, sb, dt, dev):
    """The persistent kernel (tile 11) on whole tiles and stages: the same
    bits as the one-tile-per-workgroup 256 x 256 kernel (tile 1), and
    within tolerance of the oracle on every output."""
    a = synth.generate(sa, dt, U1, [47, 0])
    b = synth.generate(sb, dt, U1, [47, 1])
    outs = []
    for t in (1, 11):
        plan = mm.Plan(sa, sb, dt, force_algo=mm.ALGO_GENERAL, tile=t)
        assert plan.info()["tile"] == t
        outs.append(synth.from_torch(run_plan(plan, a, b, dt, dev)))
    assert np.array_equal(outs[0].view(np.uint16), outs[1].view(np.uint16))
    rep = check(outs[1], oracle.matmul(a, b, dt), dt, sa[-1], abs_max(a, dt), abs_max(b, dt))
    assert rep.ok, str(rep)


def test_constant_b_tail_split(dev):
    """Constant B under the two-launch column split of a large BF16 product
    (both column ranges prepacked, each for its own tile)."""
    dt = mm.BFLOAT16
    sa, sb = (16, 512, 64), (64, 11008)
    a = synth.generate(sa, dt, ("int",), [43, 0])
    b = synth.generate(sb, dt, ("int",), [43, 1])
    plan = mm.Plan(sa, sb, dt)
    assert plan.info()["tail_col"] > 0
    plan.set_constant_b(synth.as_torch(b, dt).to(dev))
    assert plan.info()["constant_b_packed"] == 1
    Yc = _sentinel(plan.output_shape, dt, dev)
    plan.execute_constant_b(synth.as_torch(a, dt).to(dev), Yc)
    Ye = run_plan(plan, a, b, dt, dev)
    torch.cuda.synchronize()
    assert np.array_equal(synth.from_torch(Yc), synth.from_torch(Ye))


# ------------------------------------------------------------ Gemm

GEMM_DTYPES = [mm.FLOAT, mm.FLOAT16, mm.BFLOAT16]
GEMM_TRANS = [(0, 0), (1, 0), (0, 1), (1, 1)]
GEMM_LAYOUTS = [None, (), ("N",), ("M", 1), ("M", "N")]


def _cs(layout, M, N):
    return None if layout is None else tuple(M if d == "M" else N if d == "N" else d for d in layout)


def gemm_parity(M, N, K, dt, ta, tb, layout, dev, algo=0, alpha=0.75, beta=-1.5, dist=U1, seed=0, exact=False,
                offset=0, tile=0):
    sa = (K, M) if ta else (M, K)
    sb = (N, K) if tb else (K, N)
    cs = _cs(layout, M, N)
    a = synth.generate(sa, dt, dist, [seed, 0])
    b = synth.generate(sb, dt, dist, [seed, 1])
    c = None if cs is None else synth.generate(cs, dt, dist, [seed, 2])
    plan = mm.GemmPlan(sa, sb, dt, ta, tb, cs, alpha, beta, force_algo=algo, tile=tile)
    if algo:
        assert plan.algo == algo
    if tile:
        assert plan.info()["tile"] == tile

    def dev_tensor(x, shape):
        # `offset` elements past the allocation start: unaligned operands
        t = torch.empty(int(np.prod(shape)) + offset, dtype=mm.torch_dtype(dt), device=dev)[offset:].view(shape)
        t.copy_(synth.as_torch(x, dt).reshape(shape).to(dev))
        return t

    A, B = dev_tensor(a, sa), dev_tensor(b, sb)
    C = None if c is None else dev_tensor(c, cs)
    Y = torch.full((M * N + offset,), float("nan"), dtype=mm.torch_dtype(dt), device=dev)[offset:].view(M, N)
    plan.execute(A, B, Y, C)
    torch.cuda.synchronize()
    o = oracle.gemm(a, b, dt, bool(ta), bool(tb), c, alpha, beta)
    cmax = 0.0 if c is None else abs_max(c, dt)
    tol = gemm_tolerance(K, abs_max(a, dt), abs_max(b, dt), cmax, alpha, beta)
    rep = check(synth.from_torch(Y), o, dt, K, abs_max(a, dt), abs_max(b, dt), exact=exact, tol=tol)
    assert rep.ok, f"Gemm {sa} {sb} ta={ta} tb={tb} C={cs} {DT_IDS[dt]} {mm.ALGO_NAMES[plan.algo]}: {rep}"
    return plan


@pytest.mark.parametrize("dt", GEMM_DTYPES, ids=DT_IDS.get)
@pytest.mark.parametrize("ta,tb", GEMM_TRANS, ids=lambda t: f"t{t}")
@pytest.mark.parametrize("algo", [mm.ALGO_DIRECT, mm.ALGO_SPLIT_K, mm.ALGO_GENERAL], ids=lambda a: mm.ALGO_NAMES[a])
def test_gemm(dt, ta, tb, algo, dev):
    """Gemm with every transpose combination, every C layout (none, scalar,
    per column, per row, full) and each algorithm, on ragged sizes."""
    for i, layout in enumerate(GEMM_LAYOUTS):
        gemm_parity(300, 200, 520, dt, ta, tb, layout, dev, algo=algo, seed=60 + i)


@pytest.mark.parametrize("dt", GEMM_DTYPES, ids=DT_IDS.get)
@pytest.mark.parametrize("ta,tb", GEMM_TRANS, ids=lambda t: f"t{t}")
def test_gemm_every_tile(dt, ta, tb, dev):
    """Every tile entry that has Gemm kernels, general and split-K, bit-exact
    on small-integer inputs with integer alpha / beta and a per-column C;
    the other entries are refused at plan creation."""
    n_tiles = len(mm.tile_configs(dt))
    ran = 0
    for tile in range(1, n_tiles + 1):
        try:
            mm.GemmPlan((130, 1000), (1000, 70), dt, False, False, (70,), 1.0, 1.0, force_algo=mm.ALGO_GENERAL, tile=tile)
        except mm.MMError as e:
            assert e.status == mm.ERR_BAD_OPTION
            continue
        gemm_parity(130, 70, 1000, dt, ta, tb, ("N",), dev, algo=mm.ALGO_GENERAL, tile=tile, alpha=2.0, beta=-3.0,
                    dist=("int",), exact=True, seed=80 + tile)
        gemm_parity(130, 70, 1000, dt, ta, tb, ("N",), dev, algo=mm.ALGO_SPLIT_K, tile=tile, alpha=2.0, beta=-3.0,
                    dist=("int",), exact=True, seed=90 + tile)
        ran += 1
    assert ran == (6 if dt != mm.FLOAT else 5)


@pytest.mark.parametrize("dt", GEMM_DTYPES, ids=DT_IDS.get)
@pytest.mark.parametrize("ta,tb", GEMM_TRANS, ids=lambda t: f"t{t}")
def test_gemm_exact_unaligned_and_zero_k(dt, ta, tb, dev):
    """Small-integer inputs with integer alpha / beta are bit-exact; operands
    one element off 16-byte alignment take the element-wise kernel; K == 0
    gives beta * C without reading A or B."""
    gemm_parity(130, 70, 1000, dt, ta, tb, ("M", "N"), dev, algo=mm.ALGO_GENERAL, alpha=2.0, beta=-3.0,
                dist=("int",), exact=True, seed=70)
    gemm_parity(130, 70, 1000, dt, ta, tb, ("N",), dev, algo=mm.ALGO_SPLIT_K, alpha=2.0, beta=-3.0,
                dist=("int",), exact=True, seed=71)
    gemm_parity(96, 64, 256, dt, ta, tb, ("M", 1), dev, algo=mm.ALGO_GENERAL, seed=72, offset=1)
    M, N = 33, 17
    sa, sb, cs = ((0, M) if ta else (M, 0)), ((N, 0) if tb else (0, N)), (M, 1)
    a0 = synth.generate(sa, dt, U1, [73, 0])
    b0 = synth.generate(sb, dt, U1, [73, 1])
    c = synth.generate(cs, dt, U1, [73, 2])
    plan = mm.GemmPlan(sa, sb, dt, ta, tb, cs, 0.5, -2.0)
    assert plan.algo == mm.ALGO_DIRECT
    Y = _sentinel((M, N), dt, dev)
    Cd = synth.as_torch(c, dt).to(dev)
    plan.execute_ptr(0, 0, Y.data_ptr(), torch.cuda.current_stream().cuda_stream, Cd.data_ptr())
    torch.cuda.synchronize()
    o = oracle.gemm(a0, b0, dt, bool(ta), bool(tb), c, 0.5, -2.0)
    rep = check(synth.from_torch(Y), o, dt, 0, 0.0, 0.0, tol=gemm_tolerance(0, 0.0, 0.0, abs_max(c, dt), 0.5, -2.0))
    assert rep.ok, str(rep)


@pytest.mark.parametrize("ta,tb,layout", [(0, 1, ("N",)), (1, 0, ("M", "N")), (1, 1, ("M", 1)), (0, 0, ())],
                         ids=["t01-colbias", "t10-fullC", "t11-rowbias", "t00-scalar"])
def test_gemm_tail_split(ta, tb, layout, dev):
    """Last-round balancing for Gemm: columns [0, tail_col) run with the
    plan's tile and the rest with the tail tile, with B (or the rows of a
    transposed B) and a per-column or full C moved to the second launch's
    first column.  Small-integer inputs and integer alpha / beta: the result
    equals, bit for bit, each column range of a single launch forced to the
    corresponding tile, and the oracle exactly on outputs around the
    boundary."""
    dt = mm.BFLOAT16
    M, N, K = 8192, 11000, 128
    sa = (K, M) if ta else (M, K)
    sb = (N, K) if tb else (K, N)
    cs = _cs(layout, M, N)
    a = synth.generate(sa, dt, ("int",), [32, 0])
    b = synth.generate(sb, dt, ("int",), [32, 1])
    c = synth.generate(cs, dt, ("int",), [32, 2])
    plan = mm.GemmPlan(sa, sb, dt, ta, tb, cs, 2.0, -1.0)
    inf = plan.info()
    assert plan.algo == mm.ALGO_GENERAL and inf["tail_col"] > 0, inf
    cut = inf["tail_col"]
    A, B, C = (synth.as_torch(x, dt).to(dev) for x in (a, b, c))

    def run(p):
        Y = _sentinel((M, N), dt, dev)
        p.execute(A, B, Y, C)
        torch.cuda.synchronize()
        return synth.from_torch(Y)

    y = run(plan)
    ym = run(mm.GemmPlan(sa, sb, dt, ta, tb, cs, 2.0, -1.0, force_algo=mm.ALGO_GENERAL, tile=inf["tile"]))
    yr = run(mm.GemmPlan(sa, sb, dt, ta, tb, cs, 2.0, -1.0, force_algo=mm.ALGO_GENERAL, tile=inf["tail_tile"]))
    assert np.array_equal(y[:, :cut], ym[:, :cut])
    assert np.array_equal(y[:, cut:], yr[:, cut:])
    rng = np.random.default_rng(4)
    rows = rng.integers(0, M, 400)
    cols = np.concatenate([rng.integers(0, N, 200), rng.integers(cut - 8, min(N, cut + 8), 200)])
    idx = np.unique(rows * N + cols)
    o = oracle.gemm_at(a, b, dt, idx, bool(ta), bool(tb), c, 2.0, -1.0)
    rep = check(y.reshape(-1)[idx], o, dt, K, abs_max(a, dt), abs_max(b, dt), exact=True)
    assert rep.ok, str(rep)


def test_gemm_linear_layer_full_size(dev):
    """The transformer projection as a linear layer: Y = X W^T + b with
    X [8192, 4096], W [11008, 4096] (stored [N, K]) and a per-column bias, in
    BF16, checked on sampled outputs."""
    dt = mm.BFLOAT16
    M, N, K = 8192, 11008, 4096
    x = synth.generate((M, K), dt, ("normal", 0.02), [80, 0])
    w = synth.generate((N, K), dt, ("normal", 0.02), [80, 1])
    bias = synth.generate((N,), dt, ("normal", 0.02), [80, 2])
    plan = mm.GemmPlan((M, K), (N, K), dt, False, True, (N,), 1.0, 1.0)
    print(f"\n[full-size] Gemm linear layer {mm.ALGO_NAMES[plan.algo]} tile {plan.info()['tile']}", flush=True)
    Y = _sentinel((M, N), dt, dev)
    plan.execute(synth.as_torch(x, dt).to(dev), synth.as_torch(w, dt).to(dev), Y, synth.as_torch(bias, dt).to(dev))
    torch.cuda.synchronize()
    assert torch.isfinite(Y.float()).all().item()
    idx = _sample_indices((M, N), 3000, np.random.default_rng(81))
    o = oracle.gemm_at(x, w, dt, idx, False, True, bias, 1.0, 1.0)
    tol = gemm_tolerance(K, abs_max(x, dt), abs_max(w, dt), abs_max(bias, dt), 1.0, 1.0)
    rep = check(synth.from_torch(Y).reshape(-1)[idx], o, dt, K, abs_max(x, dt), abs_max(w, dt), tol=tol)
    assert rep.ok, str(rep)


# ------------------------------------------------------------ full-size workloads

def _sample_indices(shape, n, rng):
    total = int(np.prod(shape, dtype=np.int64)) if len(shape) else 1
    idx = rng.choice(total, size=min(n, total), replace=False)
    # always include the first and last elements (corners of the last tile)
    return np.unique(np.concatenate([idx, [0, total - 1]]))


# Decode and prefill sizes for which the selector takes its newer paths:
# (A shape, B shape [N, K] for the Gemm cases), element type, Gemm, and
# the plan it must make (algorithm, tile entry + 1, K partitions).
SELECTED_PATHS = [
    ((1, 4096), (4096, 8704), mm.FLOAT, False, ("skinny_m", 0, 13)),      # FP32 GEMV, K in 13 chunks
    ((15, 4096), (4096, 8704), mm.FLOAT, False, ("split_k", 8, 2)),       # FP32 9..15 rows: 32-row tiles
    ((1, 16384), (16384, 8704), mm.BFLOAT16, False, ("skinny_m", 0, 29)),  # 16-bit GEMV, long K
    ((8, 16384), (16384, 8704), mm.BFLOAT16, False, ("skinny_m", 0, 29)),  # 8 rows: packed-dot 8-row instance
    ((64, 1024), (1024, 15360), mm.BFLOAT16, False, ("general", 9, 1)),    # <= 64 rows: two-group 64x64
    ((1, 4096), (4096, 21760), mm.FLOAT16, False, ("general", 12, 1)),     # <= 32 rows, 170 tiles of 32x128
    ((48, 4096), (4096, 28672), mm.BFLOAT16, False, ("general", 14, 1)),   # <= 64 rows: 64x128
    ((16, 4096), (4096, 65536), mm.FLOAT16, False, ("general", 13, 1)),    # one full round of 32x256
    ((64, 4096), (4096, 11008), mm.BFLOAT16, False, ("split_k", 14, 2)),   # 64x128 chunks, one per CU
    ((16, 14336), (14336, 4096), mm.FLOAT16, False, ("split_k", 12, 8)),   # 32x128 chunks of a long K
    ((8, 5120), (5120, 13824), mm.BFLOAT16, False, ("split_k", 12, 2)),    # <= 32 rows, 216 64-col tiles
    ((16, 4096), (4096, 11008), mm.FLOAT, False, ("split_k", 8, 2)),       # FP32 <= 32 rows: 32x128 tiles
    ((32, 4096), (4096, 40000), mm.FLOAT, False, ("general", 8, 1)),
    ((24, 4096), (11008, 4096), mm.FLOAT, True, ("split_k", 8, 2)),        # FP32 linear layer, 24 rows
    ((16, 4096), (4096, 11008), mm.DOUBLE, False, ("split_k", 3, 8)),      # DOUBLE few rows: 32x128 tiles
    ((256, 4096), (4096, 4352), mm.BFLOAT16, False, ("split_k", 6, 4)),   # split-K tiles at most 128x128
    ((32, 4096), (11008, 4096), mm.BFLOAT16, True, ("split_k", 14, 4)),   # Gemm decode: 64x128 chunks
    ((16, 14336), (4096, 14336), mm.FLOAT16, True, ("split_k", 14, 8)),
    ((128, 16384), (8704, 16384), mm.FLOAT16, True, ("split_k", 6, 4)),
    ((1024, 4096), (4096, 11008), mm.BFLOAT16, False, ("general", 1, 1)),  # timed choice: 256x256, one round
    ((768, 4096), (4096, 4096), mm.FLOAT16, False, ("general", 3, 1)),     # three-stage 128x128
    ((512, 4096), (4096, 11008), mm.BFLOAT16, False, ("general", 2, 1)),   # 256x128
    ((128, 2048), (2048, 2048), mm.FLOAT, False, ("split_k", 6, 4)),       # FP32 split tile filling the CUs
    ((256, 4096), (4096, 11008), mm.FLOAT, False, ("general", 6, 1)),      # FP32 timed choice: no split
    ((2048, 14336), (14336, 4096), mm.BFLOAT16, False, ("split_k", 1, 2)),  # long K on 256x256 tiles
    ((1024, 14336), (4096, 14336), mm.FLOAT16, True, ("split_k", 1, 4)),    # the same for a Gemm (B transposed)
]


@pytest.mark.parametrize("sa,sb,dt,gemm,want", SELECTED_PATHS,
                         ids=lambda v: "x".join(map(str, v)) if isinstance(v, tuple) and isinstance(v[0], int) else None)
def test_selected_paths_full_size(sa, sb, dt, gemm, want, dev):
    """The selector's plan for each shape, run at full size and checked on
    sampled outputs against the oracle (Gemm: transposed B and a bias)."""
    print(f"\n[selected] {sa} x {sb} {DT_IDS[dt]} gemm={gemm}", flush=True)
    a = synth.generate(sa, dt, U1, [71, 0])
    b = synth.generate(sb, dt, U1, [71, 1])
    A = synth.as_torch(a, dt).to(dev)
    B = synth.as_torch(b, dt).to(dev)
    M, K = sa
    N = sb[0] if gemm else sb[1]
    rng = np.random.default_rng(71)
    idx = _sample_indices((M, N), 2000, rng)
    Y = _sentinel((M, N), dt, dev)
    if gemm:
        c = synth.generate((N,), dt, U1, [71, 2])
        plan = mm.GemmPlan(sa, sb, dt, False, True, (N,), 1.0, 1.0)
        plan.execute(A, B, Y, synth.as_torch(c, dt).to(dev))
        o = oracle.gemm_at(a, b, dt, idx, False, True, c, 1.0, 1.0)
        tol = gemm_tolerance(K, abs_max(a, dt), abs_max(b, dt), abs_max(c, dt), 1.0, 1.0)
    else:
        plan = mm.Plan(sa, sb, dt)
        plan.execute(A, B, Y)
        o = oracle.matmul_at(a, b, dt, idx)
        tol = None
    torch.cuda.synchronize()
    inf = plan.info()
    assert (mm.ALGO_NAMES[inf["algo"]], inf["tile"], inf["split_k"]) == want
    assert torch.isfinite(Y.float()).all().item()
    y = synth.from_torch(Y).reshape(-1)[idx]
    rep = check(y, o, dt, K, abs_max(a, dt), abs_max(b, dt), tol=tol)
    assert rep.ok, f"{sa} x {sb} {DT_IDS[dt]} {want}: {rep}"


def _leading_blocks(sa, sb):
    """(A slice, B slice) pairs that cover the output in blocks along its
    leading batch axis (one block when the output has no batch axis)."""
    ra, rb = len(sa), len(sb)
    nb = max(ra - 2 if ra > 1 else 0, rb - 2 if rb > 1 else 0)
    if nb == 0:
        return [(slice(None), slice(None))], None
    da = sa[0] if ra - 2 == nb else 1
    db = sb[0] if rb - 2 == nb else 1
    n = max(da, db)
    blocks = []
    for i in range(n):
        sla = slice(i, i + 1) if (ra - 2 == nb and da > 1) else slice(None)
        slb = slice(i, i + 1) if (rb - 2 == nb and db > 1) else slice(None)
        blocks.append((sla, slb))
    return blocks, n


def full_compare(a, b, dt, y, K, exact=False):
    """Compare every output y (storage of the full output) with the oracle,
    computed block by block along the leading batch axis to bound host
    memory; returns (elements compared, worst report)."""
    blocks, n = _leading_blocks(a.shape, b.shape)
    amax, bmax = abs_max(a, dt), abs_max(b, dt)
    compared, reps = 0, []
    for i, (sla, slb) in enumerate(blocks):
        ab = a[sla] if n else a
        bb = b[slb] if n else b
        o = oracle.matmul(np.ascontiguousarray(ab), np.ascontiguousarray(bb), dt)
        yb = y[i:i + 1] if n else y
        rep = check(yb.reshape(-1), o.reshape(-1), dt, K, amax, bmax, exact=exact)
        assert rep.ok, f"block {i}: {rep}"
        compared += o.size
        reps.append(rep)
    worst = max(reps, key=lambda r: (r.max_ulp, r.max_abs_err))
    return compared, worst


@pytest.mark.parametrize("product", synth.all_products(), ids=lambda p: p.name)
def test_workload_full_size(product, dev):
    """Each workload product at full size in the configuration the benchmark
    times (the plan's own choice), every output compared with the oracle."""
    print(f"\n[full-size] {product.name} {product.a_shape} x {product.b_shape}", flush=True)
    a, b = product.make()
    dt = product.dtype
    plan = mm.Plan(product.a_shape, product.b_shape, dt)
    Y = run_plan(plan, a, b, dt, dev)
    y = synth.from_torch(Y)
    del Y
    n, rep = full_compare(a, b, dt, y, product.K)
    print(f"[full-size] {product.name} algo={mm.ALGO_NAMES[plan.algo]} compared={n} worst block: {rep}", flush=True)
    assert n == plan.output_numel


@pytest.mark.parametrize("name", ["bf16_16x512x4096_by_4096x11008", "bf16_qk_4x32x2048x128_by_4x32x128x2048"])
def test_workload_full_size_small_integers(name, dev):
    """The projection and the attention-score product at full size on
    small-integer inputs: every output equals the oracle's, bit for bit."""
    product = [p for p in synth.all_products() if p.name == name][0]
    print(f"\n[full-size exact] {product.name}", flush=True)
    a, b = product.make(("int",))
    dt = product.dtype
    plan = mm.Plan(product.a_shape, product.b_shape, dt)
    y = synth.from_torch(run_plan(plan, a, b, dt, dev))
    n, rep = full_compare(a, b, dt, y, product.K, exact=True)
    print(f"[full-size exact] {product.name} algo={mm.ALGO_NAMES[plan.algo]} compared={n}: {rep}", flush=True)
    assert n == plan.output_numel
