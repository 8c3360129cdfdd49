"""GPU parity of MatMulInteger (page "Gemm and MatMul Performance Roadmap",
section "Remaining pull-request sequence", Roadmap PR09.1): the HIP kernels
behind mm_int_plan_create / mm_int_execute against the CPU oracle's exact
integer sums reduced modulo 2^32.  Integer results have exactly one correct
value, so every comparison is bit-exact: all four operand signedness
combinations, no / scalar / per-row (A) / per-column (B) zero points, both
kernels (direct and tiled) and every tile entry, ragged sizes, broadcast and
folded batches, rank-one operands, empty and K == 0 outputs, the cases the
tiled kernel hands to the direct one (K or N not a multiple of 16, operands
off 16-byte alignment), accumulator wrap-around, and the full-size quantized
transformer projection on sampled outputs.
"""
import numpy as np
import pytest

import oracle
from onnx_broadcast_matmul_amd import binding as mm
from onnx_broadcast_matmul_amd import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

SENTINEL = 0x5EADBEEF  # an output the kernels never write keeps this value
SIGN = {"u8": False, "s8": True}
CODE = {False: mm.UINT8, True: mm.INT8}
ZP = {"none": mm.ZP_NONE, "scalar": mm.ZP_SCALAR, "vector": mm.ZP_VECTOR}


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    mm.lib()  # the native library must load: no fallback exists
    return torch.device("cuda:0")


def _device(x, dev, offset=0):
    """Device copy of a uint8 / int8 array, starting `offset` bytes into its
    allocation (offset 1 takes the operand off 16-byte alignment)."""
    t = torch.from_numpy(np.ascontiguousarray(x).reshape(-1))
    buf = torch.empty(t.numel() + offset, dtype=t.dtype, device=dev)
    buf[offset:] = t.to(dev)
    return buf[offset:].view(x.shape)


def _zero_point(kind, signed, n, seed):
    if kind == "none":
        return None
    return synth.generate_int(() if kind == "scalar" else (n,), signed, seed)


def int_run(plan, a, b, za, zb, dev, a_off=0, b_off=0):
    Y = torch.full(plan.output_shape, SENTINEL, dtype=torch.int32, device=dev)
    plan.execute(_device(a, dev, a_off), _device(b, dev, b_off), Y,
                 None if za is None else _device(np.atleast_1d(za), dev).view(za.shape),
                 None if zb is None else _device(np.atleast_1d(zb), dev).view(zb.shape))
    torch.cuda.synchronize()
    return Y.cpu().numpy()


def int_parity(sa, sb, ta, tb, zka, zkb, dev, algo=0, tile=0, seed=0, a_off=0, b_off=0, split=0):
    sa_, sb_ = SIGN[ta], SIGN[tb]
    a = synth.generate_int(sa, sa_, [seed, 0])
    b = synth.generate_int(sb, sb_, [seed, 1])
    m = 1 if len(sa) == 1 else sa[-2]
    n = 1 if len(sb) == 1 else sb[-1]
    za = _zero_point(zka, sa_, m, [seed, 2])
    zb = _zero_point(zkb, sb_, n, [seed, 3])
    plan = mm.IntPlan(sa, sb, CODE[sa_], CODE[sb_], ZP[zka], ZP[zkb], force_algo=algo, tile=tile, split_k=split)
    if algo:
        assert plan.algo == algo
    y = int_run(plan, a, b, za, zb, dev, a_off, b_off)
    o = oracle.matmul_integer(a, b, za, zb)
    assert y.shape == o.shape
    bad = np.flatnonzero(y.reshape(-1) != o.reshape(-1))
    assert bad.size == 0, (f"{sa} x {sb} {ta}{tb} zp {zka}/{zkb} algo={mm.ALGO_NAMES[plan.algo]} "
                           f"tile={plan.info()['tile']}: {bad.size} of {o.size} differ, first at {bad[:5]}: "
                           f"{y.reshape(-1)[bad[:5]]} vs {o.reshape(-1)[bad[:5]]}")
    return plan


TYPES = [("u8", "u8"), ("u8", "s8"), ("s8", "u8"), ("s8", "s8")]
ZPS = [("none", "none"), ("scalar", "vector"), ("vector", "scalar")]


@pytest.mark.parametrize("ta,tb", TYPES, ids=lambda t: t)
@pytest.mark.parametrize("zka,zkb", ZPS, ids=lambda z: z)
@pytest.mark.parametrize("algo", [mm.ALGO_DIRECT, mm.ALGO_GENERAL], ids=lambda a: mm.ALGO_NAMES[a])
def test_int_signedness_and_zero_points(ta, tb, zka, zkb, algo, dev):
    """Broadcast batches [2,1] x [3] over ragged M, several N tiles, and a K
    that leaves the last 128-byte stage partly padded."""
    int_parity((2, 1, 200, 400), (3, 400, 272), ta, tb, zka, zkb, dev, algo=algo, seed=1)


@pytest.mark.parametrize("tile", [1, 2, 3, 4, 5])
@pytest.mark.parametrize("ta,tb", [("u8", "s8"), ("s8", "u8")], ids=lambda t: t)
def test_int_every_tile(tile, ta, tb, dev):
    int_parity((700, 1024), (1024, 600), ta, tb, "vector", "vector", dev, algo=mm.ALGO_GENERAL, tile=tile, seed=2)
    int_parity((700, 1024), (1024, 600), ta, tb, "none", "none", dev, algo=mm.ALGO_GENERAL, tile=tile, seed=3)


def test_int_folded_batch_per_row_zero_point(dev):
    """B shared by every batch: A's batches fold into the rows of one
    product, and A's per-row zero point repeats every M rows."""
    p = int_parity((4, 96, 256), (256, 160), "u8", "u8", "vector", "vector", dev, seed=4)
    assert p.info()["folded"] and p.info()["kernel_m"] == 384 and p.algo == mm.ALGO_GENERAL


@pytest.mark.parametrize("case", ["k200", "n100", "a_off", "b_off"])
def test_int_direct_handoff(case, dev):
    """Plans for the tiled kernel whose operands it cannot stream (K or N not
    a multiple of 16, A or B off 16-byte alignment) run the direct kernel."""
    sa, sb, ao, bo = (300, 512), (512, 256), 0, 0
    if case == "k200":
        sa, sb = (300, 200), (200, 256)
    elif case == "n100":
        sb = (512, 100)
    elif case == "a_off":
        ao = 1
    else:
        bo = 1
    int_parity(sa, sb, "s8", "u8", "scalar", "vector", dev, algo=mm.ALGO_GENERAL, seed=5, a_off=ao, b_off=bo)


def test_int_rank_one_empty_zero_k(dev):
    int_parity((1000,), (1000, 320), "u8", "s8", "scalar", "vector", dev, seed=6)
    int_parity((3, 130, 512), (512,), "s8", "s8", "vector", "scalar", dev, seed=7)
    int_parity((512,), (512,), "u8", "u8", "vector", "vector", dev, seed=8)
    for sa, sb in (((0, 64), (64, 32)), ((5, 64), (64, 0)), ((64, 0), (0, 32)), ((2, 3, 0), (0, 7))):
        int_parity(sa, sb, "u8", "s8", "scalar", "scalar", dev, seed=9)


@pytest.mark.parametrize("algo", [mm.ALGO_GENERAL, mm.ALGO_SPLIT_K], ids=lambda a: mm.ALGO_NAMES[a])
def test_int_wraps_modulo_2_32(algo, dev):
    """Sums beyond the INT32 range wrap: 16384 * 2^18 = 2^32 gives 0 in the
    matrix-core accumulator itself (split-K: in the partials' sum);
    255 * 255 * 40000 - 2^32 comes from the UINT8 corrections."""
    K = 1 << 18
    a = np.full((64, K), -128, np.int8)
    b = np.full((K, 64), -128, np.int8)
    plan = mm.IntPlan(a.shape, b.shape, mm.INT8, mm.INT8, force_algo=algo)
    assert plan.algo == algo
    y = int_run(plan, a, b, None, None, dev)
    assert oracle.matmul_integer_at(a, b, [0, 4095])[0] == 0 and not y.any()
    K = 40000
    a = np.full((64, K), 255, np.uint8)
    b = np.full((K, 64), 255, np.uint8)
    plan = mm.IntPlan(a.shape, b.shape, mm.UINT8, mm.UINT8, force_algo=algo)
    y = int_run(plan, a, b, None, None, dev)
    want = 255 * 255 * K - 2**32
    assert oracle.matmul_integer_at(a, b, [7])[0] == want and (y == want).all()


@pytest.mark.parametrize("ta,tb", TYPES, ids=lambda t: t)
@pytest.mark.parametrize("zka,zkb", ZPS, ids=lambda z: z)
def test_int_split_k(ta, tb, zka, zkb, dev):
    """Split-K (INT32 partials, summed modulo 2^32): each partition applies
    the zero-point and sign-flip terms of its own K range, the last one with
    a partly padded 128-byte stage; broadcast batches, ragged M and N."""
    p = int_parity((2, 1, 200, 1040), (3, 1040, 272), ta, tb, zka, zkb, dev, algo=mm.ALGO_SPLIT_K, split=3, seed=11)
    assert p.info()["split_k"] == 3 and p.info()["tile"] == 2
    # at most 64 rows: the three-stage 64 x 128 entry
    p = int_parity((2, 1, 40, 1040), (3, 1040, 272), ta, tb, zka, zkb, dev, algo=mm.ALGO_SPLIT_K, split=3, seed=12)
    assert p.info()["split_k"] == 3 and p.info()["tile"] == 4


@pytest.mark.parametrize("split", [2, 5, 8, 16, 31])
def test_int_split_counts(split, dev):
    p = int_parity((37, 4096), (4096, 272), "u8", "s8", "vector", "vector", dev, algo=mm.ALGO_SPLIT_K, split=split,
                   seed=12 + split)
    assert split // 2 < p.info()["split_k"] <= split


@pytest.mark.parametrize("sa,sb,algo,tile", [
    ((16, 4096), (4096, 11008), mm.ALGO_SPLIT_K, 4),
    ((1, 11008), (11008, 4096), mm.ALGO_SPLIT_K, 4),
    ((2, 8, 4096), (2, 4096, 2048), mm.ALGO_SPLIT_K, 4),
    ((48, 4096), (4096, 28672), mm.ALGO_GENERAL, 4),   # one round of 64 x 128 tiles, whole
    ((128, 8192), (8192, 8192), mm.ALGO_SPLIT_K, 5),   # 64 tiles x 4 chunks: the three-stage 128 x 128 entry
])
def test_int_few_rows(sa, sb, algo, tile, dev):
    """The plans' own choices for few-row quantized layers, every output
    compared."""
    p = int_parity(sa, sb, "u8", "s8", "scalar", "vector", dev, seed=13)
    assert p.algo == algo and p.info()["tile"] == tile


@pytest.mark.parametrize("ta,tb,zka,zkb", [("u8", "s8", "scalar", "vector"), ("s8", "u8", "vector", "vector")],
                         ids=["u8s8", "s8u8"])
def test_int_tail_split(ta, tb, zka, zkb, dev):
    """Last-round balancing: columns [0, tail_col) run with the plan's tile
    and the rest with the tail tile, B, Y and a per-column B zero point
    moved by tail_col columns.  The result equals single launches forced to
    either tile and the oracle on outputs around the boundary."""
    sa, sb = (16, 512, 256), (256, 11008)
    sa_, sb_ = SIGN[ta], SIGN[tb]
    a = synth.generate_int(sa, sa_, [33, 0])
    b = synth.generate_int(sb, sb_, [33, 1])
    za = _zero_point(zka, sa_, 512, [33, 2])
    zb = _zero_point(zkb, sb_, 11008, [33, 3])
    plan = mm.IntPlan(sa, sb, CODE[sa_], CODE[sb_], ZP[zka], ZP[zkb])
    inf = plan.info()
    assert plan.algo == mm.ALGO_GENERAL and inf["tail_col"] > 0, inf
    cut = inf["tail_col"]
    y = int_run(plan, a, b, za, zb, dev).reshape(-1, 11008)
    for t in (inf["tile"], inf["tail_tile"]):
        single = mm.IntPlan(sa, sb, CODE[sa_], CODE[sb_], ZP[zka], ZP[zkb], force_algo=mm.ALGO_GENERAL, tile=t)
        ys = int_run(single, a, b, za, zb, dev).reshape(-1, 11008)
        part = slice(0, cut) if t == inf["tile"] else slice(cut, None)
        np.testing.assert_array_equal(y[:, part], ys[:, part])
    rng = np.random.default_rng(5)
    rows = rng.integers(0, 8192, 300)
    cols = np.concatenate([rng.integers(0, 11008, 150), rng.integers(cut - 8, cut + 8, 150)])
    idx = np.unique(rows * 11008 + cols)
    np.testing.assert_array_equal(y.reshape(-1)[idx], oracle.matmul_integer_at(a, b, idx, za, zb))


def test_int_full_size_projection(dev):
    """The quantized transformer projection at full size, in the
    configuration the benchmark times, on sampled outputs."""
    prod = synth.INT_PRODUCTS[0]
    a, b, za, zb = prod.make()
    plan = mm.IntPlan(prod.a_shape, prod.b_shape, CODE[prod.a_signed], CODE[prod.b_signed], prod.a_zp, prod.b_zp)
    print(f"\n[full-size] {prod.name} {mm.ALGO_NAMES[plan.algo]} tile {plan.info()['tile']}", flush=True)
    y = int_run(plan, a, b, za, zb, dev).reshape(-1)
    rng = np.random.default_rng(90)
    idx = np.unique(np.concatenate([rng.choice(y.size, 3000, replace=False), [0, y.size - 1]]))
    o = oracle.matmul_integer_at(a, b, idx, za, zb)
    np.testing.assert_array_equal(y[idx], o)
    assert not (y == SENTINEL).any()
