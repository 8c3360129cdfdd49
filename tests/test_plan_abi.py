"""CPU tests of the C ABI: exported symbols, shape resolution against numpy,
every error path, broadcast strides / collapse / fold, and the algorithm
selector.  Plan creation makes no GPU call, so none of this needs a GPU."""
import ctypes
import itertools
import os
import re

import numpy as np
import pytest

from onnx_broadcast_matmul_amd import binding as mm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not os.path.exists(mm.LIB_PATH):
        from onnx_broadcast_matmul_amd import build

        build.build()
    return mm.lib()


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "mm.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*[\w\s\*]*?\b(mm_\w+)\s*\(", text, flags=re.M)))


def test_header_symbols_exported():
    names = _declared_functions()
    assert "mm_plan_create" in names and "mm_execute" in names and len(names) >= 13
    lib = ctypes.CDLL(mm.LIB_PATH)
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing


def _try_plan(sa, sb, dtype=mm.FLOAT, **kw):
    try:
        return mm.Plan(sa, sb, dtype, **kw), None
    except mm.MMError as e:
        return None, e.status


def test_output_shapes_match_numpy_exhaustive():
    dims = (0, 1, 2, 3)
    shapes = [s for r in range(1, 5) for s in itertools.product(dims, repeat=r)]
    zeros = {s: np.zeros(s, dtype=np.float32) for s in shapes}
    for sa in shapes:
        for sb in shapes:
            try:
                want = np.matmul(zeros[sa], zeros[sb]).shape
            except ValueError:
                want = None
            plan, st = _try_plan(sa, sb)
            if want is None:
                assert plan is None and st in (mm.ERR_K_MISMATCH, mm.ERR_BROADCAST), (sa, sb, st)
            else:
                assert plan is not None, (sa, sb, st)
                assert plan.output_shape == want, (sa, sb)
                assert plan.output_numel == int(np.prod(want, dtype=np.int64))
                n = plan.output_numel
                assert plan.algo == (mm.ALGO_EMPTY if n == 0 else mm.ALGO_ZERO_FILL if sa[-1] == 0 else plan.algo)


@pytest.mark.parametrize("sa,sb,dtype,status", [
    ((), (3, 4), mm.FLOAT, mm.ERR_RANK),
    ((3, 4), (), mm.FLOAT, mm.ERR_RANK),
    ((1,) * 11, (1, 1), mm.FLOAT, mm.ERR_RANK),
    ((2, -1), (3, 4), mm.FLOAT, mm.ERR_NEG_DIM),
    ((2, 3), (3, -4), mm.FLOAT, mm.ERR_NEG_DIM),
    ((2, 3), (4, 5), mm.FLOAT, mm.ERR_K_MISMATCH),
    ((2, 2, 3), (3, 3, 4), mm.FLOAT, mm.ERR_BROADCAST),
    ((0, 2, 3), (2, 3, 4), mm.FLOAT, mm.ERR_BROADCAST),
    ((2, 3), (3, 4), 7, mm.ERR_DTYPE),
    ((2, 3), (3, 4), 12, mm.ERR_DTYPE),
])
def test_plan_errors(sa, sb, dtype, status):
    plan, st = _try_plan(sa, sb, dtype)
    assert plan is None and st == status
    assert mm.lib().mm_last_error()


def test_rank_limit_accepts_eight_batch_dims():
    plan, st = _try_plan((2,) * 8 + (3, 4), (4, 5))
    assert st is None and plan.output_shape == (2,) * 8 + (3, 5)


@pytest.mark.parametrize("kw,status", [
    (dict(force_algo=mm.ALGO_EMPTY), mm.ERR_BAD_OPTION),
    (dict(force_algo=99), mm.ERR_BAD_OPTION),
    (dict(force_algo=mm.ALGO_GENERAL, tile=99), mm.ERR_BAD_OPTION),
    (dict(force_algo=mm.ALGO_SPLIT_K, split_k=-1), mm.ERR_BAD_OPTION),
])
def test_option_errors(kw, status):
    plan, st = _try_plan((64, 64), (64, 64), mm.FLOAT, **kw)
    assert plan is None and st == status


def test_reserved_option_rejected():
    L = mm.lib()
    h = ctypes.c_void_p()
    opt = mm.PlanOptions(0, 0, 0, 1)
    st = L.mm_plan_create_ex(mm._shape((4, 4)), 2, mm._shape((4, 4)), 2, mm.FLOAT, ctypes.byref(opt),
                             ctypes.byref(h))
    assert st == mm.ERR_BAD_OPTION and not h.value


def test_null_arguments():
    L = mm.lib()
    st = L.mm_plan_create(mm._shape((4, 4)), 2, mm._shape((4, 4)), 2, mm.FLOAT, None)
    assert st == mm.ERR_NULL_ARG
    assert L.mm_execute(None, None, None, None, None) == mm.ERR_NULL_ARG
    assert L.mm_plan_output_numel(None) == -1
    assert L.mm_plan_algo(None) == -1
    L.mm_plan_destroy(None)  # NULL is ignored
    shp = (ctypes.c_int64 * mm.MAX_RANK)()
    rank = ctypes.c_int()
    assert L.mm_plan_output_shape(None, shp, ctypes.byref(rank)) == mm.ERR_NULL_ARG


def test_execute_without_gpu_paths():
    """Empty outputs launch nothing (NULL pointers allowed); a non-empty
    output with NULL pointers is refused before any GPU call."""
    empty = mm.Plan((3, 0, 5), (5, 4), mm.FLOAT)
    assert empty.algo == mm.ALGO_EMPTY
    empty.execute_ptr(0, 0, 0)
    zero_k = mm.Plan((3, 4, 0), (0, 5), mm.FLOAT)
    assert zero_k.algo == mm.ALGO_ZERO_FILL
    with pytest.raises(mm.MMError) as e:
        zero_k.execute_ptr(0, 0, 0)
    assert e.value.status == mm.ERR_NULL_ARG
    p = mm.Plan((3, 4, 5), (5, 6), mm.FLOAT)
    with pytest.raises(mm.MMError) as e:
        p.execute_ptr(0, 0, 1 << 20)
    assert e.value.status == mm.ERR_NULL_ARG


def test_status_strings():
    L = mm.lib()
    for s in range(11):
        assert L.mm_status_string(s)


@pytest.mark.parametrize("sa,sb,dims,sa_str,sb_str,folded,kernel_m", [
    ((8, 1, 512, 512), (1, 6, 512, 512), (8, 6), (262144, 0), (0, 262144), False, 512),
    ((2, 3, 4, 5, 6), (6, 7), (), (), (), True, 120),
    ((2, 1, 5, 6), (3, 6, 7), (2, 3), (30, 0), (0, 42), False, 5),
    ((2, 3, 5, 6), (2, 3, 6, 7), (6,), (30,), (42,), False, 5),
    ((1, 1, 5, 6), (6, 7), (), (), (), False, 5),
    ((6,), (2, 3, 6, 7), (6,), (0,), (42,), False, 1),
    ((4, 1, 2, 5, 6), (3, 2, 6, 7), (4, 3, 2), (60, 0, 30), (0, 84, 42), False, 5),
    ((4, 3, 2, 5, 6), (1, 1, 6, 7), (), (), (), True, 120),
    ((4, 1, 2, 5, 6), (1, 1, 6, 7), (), (), (), True, 40),
    ((2, 5, 6), (6,), (), (), (), True, 10),
    ((16, 512, 4096), (4096, 11008), (), (), (), True, 8192),
])
def test_strides_collapse_fold(sa, sb, dims, sa_str, sb_str, folded, kernel_m):
    info = mm.Plan(sa, sb, mm.BFLOAT16).info()
    assert info["batch_dims"] == dims
    assert info["a_batch_strides"] == sa_str
    assert info["b_batch_strides"] == sb_str
    assert info["folded"] == folded
    assert info["kernel_m"] == kernel_m


def _plan_walk_matches_broadcast(sa, sb):
    """The collapsed (dims, strides) must address exactly the matrices
    numpy's broadcasting pairs up, in output batch order."""
    info = mm.Plan(sa, sb, mm.FLOAT).info()
    M, N, K = info["M"], info["N"], info["K"]
    a_idx = np.arange(int(np.prod(sa)) // (M * K) if len(sa) > 1 else 1).reshape(sa[:-2] or (1,))
    b_idx = np.arange(int(np.prod(sb)) // (K * N) if len(sb) > 1 else 1).reshape(sb[:-2] or (1,))
    bshape = np.broadcast_shapes(a_idx.shape, b_idx.shape)
    ea = np.broadcast_to(a_idx, bshape).reshape(-1) * M * K
    eb = np.broadcast_to(b_idx, bshape).reshape(-1) * K * N
    if info["folded"]:
        assert np.all(eb == 0) and np.array_equal(ea, np.arange(ea.size) * M * K)
        return
    dims = info["batch_dims"]
    oa, ob = [], []
    for idx in itertools.product(*[range(d) for d in dims]):
        oa.append(sum(i * s for i, s in zip(idx, info["a_batch_strides"])))
        ob.append(sum(i * s for i, s in zip(idx, info["b_batch_strides"])))
    if not dims:
        oa, ob = [0], [0]
    assert np.array_equal(np.array(oa), ea) and np.array_equal(np.array(ob), eb)


def test_collapsed_walk_equals_numpy_broadcast():
    dims = (1, 2, 3)
    for ra in range(2, 5):
        for rb in range(2, 5):
            for ba in itertools.product(dims, repeat=ra - 2):
                for bb in itertools.product(dims, repeat=rb - 2):
                    try:
                        np.broadcast_shapes(ba, bb)
                    except ValueError:
                        continue
                    _plan_walk_matches_broadcast(ba + (2, 3), bb + (3, 4))


SELECTOR_CASES = [
    # workload products and the algorithm the selector must pick
    ((4, 64, 96), (96, 80), mm.FLOAT, "direct"),
    ((96,), (96, 80), mm.FLOAT, "direct"),
    ((4, 64, 96), (96,), mm.FLOAT, "skinny_n"),
    ((8, 16), (16, 8), mm.FLOAT, "direct"),
    ((4, 64, 96), (96,), mm.DOUBLE, "direct"),   # no skinny-N kernel for DOUBLE: tiny stays direct
    ((32, 256), (256, 32), mm.BFLOAT16, "general"),  # 16-bit: MFMA tiles beat the direct loop from K = 64
    ((32, 16), (16, 32), mm.BFLOAT16, "direct"),
    ((8, 256, 16), (16, 256), mm.BFLOAT16, "general"),  # 2^19 outputs: the tiles win even at K = 16
    ((1, 4096), (4096, 2048), mm.FLOAT, "skinny_m"),    # FP32 GEMV over 8 column blocks: K cut into chunks
    ((8, 1024), (1024, 30720), mm.FLOAT, "skinny_m"),
    ((1, 16384), (16384, 8704), mm.BFLOAT16, "skinny_m"),  # 16-bit: up to 4 rows, long K, large B
    ((4, 4096), (4096, 30720), mm.BFLOAT16, "general"),   # 16-bit, K < 8192: the tiles
    ((8, 16384), (16384, 8704), mm.BFLOAT16, "skinny_m"),  # 16-bit, 8 rows, K >= 16384, N >= 8704
    ((8, 16384), (16384, 8192), mm.BFLOAT16, "split_k"),   # N below the measured 8704
    ((8, 16384), (16384, 8705), mm.BFLOAT16, "split_k"),   # B / Y rows not whole 16-byte chunks
    ((2, 16388), (16388, 8704), mm.FLOAT16, "split_k"),    # A rows not whole 16-byte chunks
    ((4, 8192), (8192, 8196), mm.BFLOAT16, "split_k"),     # the 4-row rule needs aligned rows too
    ((8, 16384), (16384, 4352), mm.BFLOAT16, "split_k"),   # 16-bit, 8 rows, narrower B: the tiles
    ((8, 4096), (4096, 30720), mm.FLOAT16, "general"),
    ((15, 16384), (16384, 30720), mm.FLOAT16, "general"),
    ((1, 4096), (4096, 11008), mm.BFLOAT16, "split_k"),   # 172 tiles and K >= 4096
    ((1, 1024), (1024, 11008), mm.BFLOAT16, "general"),   # 172 tiles, K < 4096
    ((15, 4096), (4096, 8704), mm.FLOAT, "split_k"),      # FP32 9..15 rows: 32-row tiles, K in chunks
    ((8, 4096), (4096, 8704), mm.FLOAT, "skinny_m"),      # FP32 up to 8 rows: the K-split GEMV
    ((15, 16384), (16384, 2048), mm.FLOAT, "split_k"),
    ((15, 1024), (1024, 8704), mm.FLOAT, "split_k"),      # FP32 <= 32 rows: 32-row tiles, K in chunks
    ((16, 4096), (4096, 8704), mm.FLOAT, "split_k"),      # 16 rows and more: never the K-split GEMV
    ((128, 4096), (4096, 10880), mm.FLOAT, "split_k"),
    ((128, 4096), (4096, 15360), mm.FLOAT, "split_k"),  # FP32 33-512 rows: the time model splits
    ((32, 16384), (16384, 21760), mm.FLOAT, "split_k"),   # 170 tiles of 32x128: two chunks
    ((32, 4096), (4096, 40000), mm.FLOAT, "general"),     # past one tile per CU: whole tiles
    ((15, 4096), (4096, 256), mm.BFLOAT16, "split_k"),
    ((4, 256), (256, 2048), mm.BFLOAT16, "general"),   # short K: the tiles
    ((256, 4096), (4096, 256), mm.FLOAT, "split_k"),
    ((4096, 256), (256, 8), mm.BFLOAT16, "general"),   # eight 16-bit columns, short K: the tiles
    ((4096, 256), (256, 4), mm.BFLOAT16, "skinny_n"),
    ((256, 4096), (4096, 8), mm.DOUBLE, "split_k"),    # no skinny kernels: few tiles and long K take split-K
    ((256, 256), (256, 256), mm.FLOAT, "direct"),    # FP32: direct up to about 2^25 FLOPs
    ((8, 128, 256), (256, 128), mm.FLOAT, "general"),
    ((1024, 1024), (1024, 1024), mm.FLOAT, "general"),
    ((8, 1, 512, 512), (1, 6, 512, 512), mm.FLOAT, "general"),
    ((16, 512, 4096), (4096, 11008), mm.BFLOAT16, "general"),
    ((32, 1, 4096), (32, 4096, 4096), mm.FLOAT16, "skinny_m"),
    ((8192, 4096), (4096, 8), mm.FLOAT16, "skinny_n"),
    ((64, 131072), (131072, 64), mm.FLOAT, "split_k"),
    ((4, 32, 2048, 128), (4, 32, 128, 2048), mm.BFLOAT16, "general"),
    ((4, 32, 2048, 2048), (4, 32, 2048, 128), mm.BFLOAT16, "general"),
    ((1024, 1024), (1024, 1), mm.FLOAT, "skinny_n"),       # N == 1 never goes to split-K
    ((1, 1 << 20), (1 << 20, 1), mm.FLOAT, "skinny_n"),
    ((3, 0, 5), (5, 4), mm.FLOAT, "empty"),
    ((3, 4, 0), (0, 5), mm.FLOAT, "zero_fill"),
]


@pytest.mark.parametrize("sa,sb,dt,algo", SELECTOR_CASES)
def test_selector(sa, sb, dt, algo):
    assert mm.ALGO_NAMES[mm.Plan(sa, sb, dt).algo] == algo


@pytest.mark.parametrize("M,K,N,algo", [
    (1, 4096, 15360, "split_k"),    # FP32 Gemm, <= 32 rows: 32-row tiles, K in chunks
    (32, 1024, 11008, "split_k"),
    (32, 4096, 21760, "split_k"),   # 170 tiles of 32 x 128: two chunks
    (32, 4096, 40000, "general"),   # past one tile per CU
    (128, 4096, 15360, "split_k"),  # 128 rows: the time model (two chunks of 128 x 128)
    (512, 2048, 2048, "general"),   # the split's gain does not cover the reduction
])
def test_fp32_gemm_few_rows(M, K, N, algo):
    g = mm.GemmPlan((M, K), (N, K), mm.FLOAT, False, True, (N,), 1.0, 1.0)
    assert mm.ALGO_NAMES[g.algo] == algo


def test_small_m_tiles():
    """16-bit products of at most 64 rows take 64 x 64 tiles with two K
    groups up to one tile per CU; beyond that, 128-column tiles one row tile
    high (32 x 128 up to 32 rows, else 64 x 128), and for at most 32 rows
    32 x 256 tiles when every round of them fills three quarters of the
    CUs.  Gemm takes its 64 x 64 entry."""
    t16 = mm.tile_configs(mm.BFLOAT16)
    assert t16[8][:2] == (64, 64) and t16[4][:2] == (64, 64)
    assert [c[:2] for c in t16[11:]] == [(32, 128), (32, 256), (64, 128)]
    for sa, sb, want in [((64, 1024), (1024, 15360), 9), ((2, 32, 1024), (2, 1024, 8192), 9),
                         ((1, 4096), (4096, 21760), 12), ((16, 4096), (4096, 30720), 12),
                         ((33, 4096), (4096, 30720), 14), ((64, 2048), (2048, 128256), 14),
                         ((16, 4096), (4096, 49152), 13),    # 192 tiles of 32 x 256: one round at 3/4
                         ((32, 4096), (4096, 65536), 13),    # 256: one full round
                         ((16, 4096), (4096, 98304), 12),    # 384: a last round of 128 tiles
                         ((16, 4096), (4096, 128256), 13),   # 501: a last round of 245
                         ((2, 16, 2048), (2, 2048, 32768), 13)]:
        inf = mm.Plan(sa, sb, mm.BFLOAT16).info()
        assert mm.ALGO_NAMES[inf["algo"]] == "general" and inf["tile"] == want, (sa, sb, inf["tile"])
        assert inf["tail_col"] == 0
    g = mm.GemmPlan((32, 4096), (21760, 4096), mm.FLOAT16, False, True, None, 1.0, 0.0)
    assert g.algo == mm.ALGO_GENERAL and g.info()["tile"] == 5
    # more rows: the time model, which leaves the small-row entries out
    for sa, sb in [((65, 4096), (4096, 21760)), ((96, 4096), (4096, 65536)), ((128, 2048), (2048, 40000))]:
        assert mm.Plan(sa, sb, mm.BFLOAT16).info()["tile"] not in (4, 5, 9, 12, 13, 14)


@pytest.mark.parametrize("sa,sb,want", [
    ((16, 4096), (4096, 11008), ("split_k", 12, 2)),   # 64 x 64 chunks would put 344 workgroups on 256 CUs
    ((48, 8192), (8192, 11008), ("split_k", 14, 2)),   # 86 tiles of 64 x 128: 2 chunks, not 3
    ((16, 14336), (14336, 4096), ("split_k", 12, 8)),  # 64 x 64 chunks of 3584: K-long
    ((64, 14336), (14336, 4096), ("split_k", 14, 8)),
    ((32, 4096), (4096, 4096), ("split_k", 5, 4)),     # 64 x 64 in 4 chunks of 1024 fill the CUs
    ((64, 8192), (8192, 4096), ("split_k", 5, 4)),
    ((16, 1024), (1024, 4096), ("split_k", 5, 4)),
    ((16, 4096), (4096, 14336), ("split_k", 12, 2)),   # <= 32 rows, up to one 64-column tile per CU: split
    ((1, 4096), (4096, 16384), ("split_k", 12, 2)),
    ((33, 4096), (4096, 14336), ("general", 9, 1)),    # more rows: the two-group 64 x 64 tiles
    ((16, 2048), (2048, 14336), ("general", 9, 1)),    # K < 4096
])
def test_small_m_split_tiles(sa, sb, want):
    """16-bit split-K of at most 64 rows: the 64 x 64 tiles unless their
    chunks overfill the CUs or stay long, then the 128-column small-row
    tile with at most one workgroup per CU."""
    for dt in (mm.BFLOAT16, mm.FLOAT16):
        inf = mm.Plan(sa, sb, dt).info()
        assert (mm.ALGO_NAMES[inf["algo"]], inf["tile"], inf["split_k"]) == want, inf


def test_small_m_entries_left_out_of_larger_products():
    """The split-K tile of a product of more than 64 rows, and the forced
    small-row tiles on any shape, work as before."""
    for sa, sb in [((96, 4096), (4096, 4096)), ((128, 8192), (8192, 2048)), ((200, 14336), (14336, 1024))]:
        inf = mm.Plan(sa, sb, mm.BFLOAT16).info()
        if mm.ALGO_NAMES[inf["algo"]] == "split_k":
            assert inf["tile"] not in (12, 13, 14), (sa, sb, inf)
    for t in (12, 13, 14):
        inf = mm.Plan((300, 520), (520, 200), mm.BFLOAT16, force_algo=mm.ALGO_GENERAL, tile=t).info()
        assert inf["tile"] == t and inf["tail_col"] == 0
        inf = mm.Plan((100, 4096), (4096, 300), mm.FLOAT16, force_algo=mm.ALGO_SPLIT_K, tile=t).info()
        assert inf["tile"] == t and inf["split_k"] >= 2


@pytest.mark.parametrize("sa,sb,want", [
    ((4096, 4096), (4096, 14336), 1),   # 3.5 rounds of 256 x 256 beat 7 rounds of 128 x 128
    ((2048, 4096), (4096, 14336), 1),
    ((1024, 4096), (4096, 11008), 1),   # 172 tiles of 256 x 256: one round
    ((1024, 4096), (4096, 4096), 3),    # 256 tiles of 128 x 128: three stages, one per CU
    ((768, 4096), (4096, 4096), 3),
    ((512, 4096), (4096, 11008), 2),    # 172 tiles of 256 x 128
    ((8192, 8192), (8192, 8192), 1),
    ((8192, 4096), (4096, 1024), 6),    # 2 x 256 tiles of 128 x 128, two per CU
])
def test_timed_tile_selection(sa, sb, want):
    """16-bit general plans of more than 64 rows take the tile entry of least
    estimated time (a launch cost plus round times per occupancy level)."""
    for dt in (mm.BFLOAT16, mm.FLOAT16):
        inf = mm.Plan(sa, sb, dt).info()
        assert mm.ALGO_NAMES[inf["algo"]] == "general" and inf["tile"] == want, (sa, sb, inf)


@pytest.mark.parametrize("sa,sb,want", [
    ((2048, 14336), (14336, 4096), ("split_k", 1, 2)),  # 128 tiles of 256 x 256, K 14336: two chunks
    ((1024, 14336), (14336, 4096), ("split_k", 1, 4)),  # 64 tiles: four chunks
    ((2048, 11008), (11008, 4096), ("split_k", 1, 2)),
    ((2048, 4096), (4096, 4096), ("general", 6, 1)),    # K 4096: the partials' round trip does not pay
    ((2048, 8192), (8192, 4096), ("general", 6, 1)),
    ((4096, 14336), (14336, 4096), ("general", 1, 1)),  # a full round of large tiles
])
def test_large_tile_split(sa, sb, want):
    """A 16-bit product that fills at most half a round of 256 x 256 tiles
    with a long K splits K on that tile when the time estimate (chunks
    filling one round plus the partials' round trip) gains 5 %."""
    for dt in (mm.BFLOAT16, mm.FLOAT16):
        inf = mm.Plan(sa, sb, dt).info()
        assert (mm.ALGO_NAMES[inf["algo"]], inf["tile"], inf["split_k"]) == want, inf
    # Gemm with a transposed B takes the same rule (its 256 x 256 entry has a split-K kernel)
    g = mm.GemmPlan((2048, 14336), (4096, 14336), mm.BFLOAT16, False, True, None, 1.0, 0.0)
    assert (g.algo, g.info()["tile"], g.info()["split_k"]) == (mm.ALGO_SPLIT_K, 1, 2)


@pytest.mark.parametrize("sa,sb,want", [
    ((128, 2048), (2048, 2048), ("split_k", 6, 4)),   # 64 x 64 tiles in 4 chunks fill the CUs
    ((128, 1024), (1024, 1024), ("split_k", 6, 4)),
    ((128, 4096), (4096, 4096), ("split_k", 7, 8)),   # 128 x 128 tiles in 8 chunks fill them too
    ((256, 4096), (4096, 11008), ("general", 6, 1)),  # 688 tiles of 64 x 64: no split
    ((64, 131072), (131072, 64), ("split_k", 6, 256)),
])
def test_fp32_split_tiles(sa, sb, want):
    """FLOAT split-K takes the two-K-group tile whose chunks fill the most
    CUs, and the split-K occupancy test counts the general path's own tiles."""
    inf = mm.Plan(sa, sb, mm.FLOAT).info()
    assert (mm.ALGO_NAMES[inf["algo"]], inf["tile"], inf["split_k"]) == want, inf


def test_tile_table():
    t16 = mm.tile_configs(mm.BFLOAT16)
    t32 = mm.tile_configs(mm.FLOAT)
    assert t16 == mm.tile_configs(mm.FLOAT16)
    # K per LDS stage: 128 or 64 bytes, so 128-byte split partitions hold whole stages
    assert all(bk in (32, 64) for _, _, bk in t16) and all(bk == 32 for _, _, bk in t32)
    assert (256, 256, 64) in t16
    for dt, table in ((mm.BFLOAT16, t16), (mm.FLOAT, t32)):
        for i in range(len(table)):
            info = mm.Plan((300, 200), (200, 100), dt, force_algo=mm.ALGO_GENERAL, tile=i + 1).info()
            assert info["tile"] == i + 1


def test_split_plan():
    info = mm.Plan((64, 1000), (1000, 64), mm.FLOAT, force_algo=mm.ALGO_SPLIT_K, split_k=3).info()
    assert info["algo_name"] == "split_k"
    assert info["k_chunk"] % 32 == 0 and info["split_k"] == 3
    assert info["k_chunk"] * (info["split_k"] - 1) < 1000 <= info["k_chunk"] * info["split_k"]
    assert info["workspace_bytes"] == 3 * 64 * 64 * 4
    # more partitions than K stages: clamped so none is empty
    info = mm.Plan((8, 100), (100, 8), mm.BFLOAT16, force_algo=mm.ALGO_SPLIT_K, split_k=50).info()
    assert info["split_k"] == 2 and info["k_chunk"] == 64
    auto = mm.Plan((64, 131072), (131072, 64), mm.FLOAT).info()
    assert auto["split_k"] >= 2 and auto["k_chunk"] >= 256


def test_info_flops_bytes():
    info = mm.Plan((8, 1, 512, 512), (1, 6, 512, 512), mm.FLOAT).info()
    assert info["flops"] == 2.0 * 48 * 512 ** 3
    assert info["min_bytes"] == 4.0 * (8 * 512 * 512 + 6 * 512 * 512 + 48 * 512 * 512)


# ---------------------------------------------------------------- DOUBLE

@pytest.mark.parametrize("sa,sb,algo", [
    ((4, 64, 96), (96, 80), mm.ALGO_DIRECT),
    ((1024, 1024), (1024, 1024), mm.ALGO_GENERAL),
    ((32, 1, 4096), (32, 4096, 4096), mm.ALGO_GENERAL),   # skinny-M shape: no FP64 skinny kernel
    ((8192, 4096), (4096, 8), mm.ALGO_SPLIT_K),           # skinny-N shape: 128 tiles, long K
    ((64, 131072), (131072, 64), mm.ALGO_SPLIT_K),
])
def test_double_plans(sa, sb, algo):
    """DOUBLE goes through the same plan as the other types; its skinny
    shapes take the tiled FP64 kernel and split-K keeps double partials."""
    plan = mm.Plan(sa, sb, mm.DOUBLE)
    assert plan.algo == algo
    inf = plan.info()
    assert inf["dtype"] == mm.DOUBLE
    if algo == mm.ALGO_SPLIT_K:
        assert inf["workspace_bytes"] == inf["split_k"] * inf["batch"] * inf["kernel_m"] * inf["N"] * 8
        assert inf["k_chunk"] % 16 == 0
    na = int(np.prod(sa)); nb = int(np.prod(sb))
    assert inf["min_bytes"] == 8.0 * (na + nb + plan.output_numel)


def test_skinny_m_k_split_plans():
    """Skinny-M cuts K into whole 64-row chunks (at most two workgroups per
    CU, at most 64 chunks) when its column workgroups are fewer than two per
    CU, and keeps one chunk, with no workspace, when they are not; a
    requested count is clamped so that every chunk holds rows."""
    p = mm.Plan((1, 4096), (4096, 2048), mm.BFLOAT16, force_algo=mm.ALGO_SKINNY_M)
    inf = p.info()
    # 2048 columns / 512 per workgroup = 4 workgroups -> 128 chunks wanted, at most 64
    assert inf["split_k"] == 64 and inf["k_chunk"] == 64
    assert inf["workspace_bytes"] == 64 * 1 * 1 * 2048 * 4 == p.workspace_bytes
    mid = mm.Plan((8, 16384), (16384, 8704), mm.FLOAT, force_algo=mm.ALGO_SKINNY_M).info()
    # 34 workgroups of 256 FP32 columns -> at most 512 / 34 = 15 chunks: 18 blocks of 64 rows each
    assert (mid["split_k"], mid["k_chunk"]) == (15, 1152)
    wide = mm.Plan((4, 4096), (4096, 131072), mm.FLOAT, force_algo=mm.ALGO_SKINNY_M).info()
    assert wide["split_k"] == 1 and wide["k_chunk"] == 4096 and wide["workspace_bytes"] == 0
    short = mm.Plan((1, 200), (200, 64), mm.FLOAT, force_algo=mm.ALGO_SKINNY_M).info()
    assert (short["split_k"], short["k_chunk"]) == (4, 64) and short["workspace_bytes"] == 4 * 64 * 4
    one = mm.Plan((1, 64), (64, 64), mm.FLOAT, force_algo=mm.ALGO_SKINNY_M).info()
    assert one["split_k"] == 1 and one["workspace_bytes"] == 0
    for req, want_chunk, want_split in [(1, 4160, 1), (7, 640, 7), (64, 128, 33), (500, 64, 65)]:
        f = mm.Plan((3, 4100), (4100, 300), mm.FLOAT16, force_algo=mm.ALGO_SKINNY_M, split_k=req).info()
        assert (f["k_chunk"], f["split_k"]) == (want_chunk, want_split)
        assert f["k_chunk"] % 64 == 0 and (f["split_k"] - 1) * f["k_chunk"] < 4100 <= f["split_k"] * f["k_chunk"]
        assert f["workspace_bytes"] == (0 if want_split == 1 else want_split * 3 * 300 * 4)
    assert _try_plan((1, 64), (64, 64), mm.FLOAT, force_algo=mm.ALGO_SKINNY_M, split_k=-1)[1] == mm.ERR_BAD_OPTION


@pytest.mark.parametrize("algo", [mm.ALGO_SKINNY_M, mm.ALGO_SKINNY_N])
def test_double_rejects_forced_skinny(algo):
    plan, st = _try_plan((64, 64), (64, 8), mm.DOUBLE, force_algo=algo)
    assert plan is None and st == mm.ERR_BAD_OPTION


def test_double_tile_table():
    assert mm.lib().mm_tile_count(mm.DOUBLE) == 3
    assert mm.tile_configs(mm.DOUBLE) == [(128, 128, 16), (64, 64, 16), (32, 128, 16)]


@pytest.mark.parametrize("sa,sb,want", [
    ((16, 4096), (4096, 11008), ("split_k", 3, 8)),   # 86 tiles of 32 x 128: 8 chunks (688 workgroups)
    ((1, 4096), (4096, 4096), ("split_k", 3, 8)),     # at most 8 chunks
    ((16, 2048), (2048, 4096), ("split_k", 3, 4)),    # at most K / 512 chunks
    ((16, 4096), (4096, 28672), ("split_k", 3, 2)),   # 224 tiles: 2 chunks
    ((16, 4096), (4096, 65536), ("general", 3, 1)),   # past one tile per CU: whole tiles
    ((33, 4096), (4096, 11008), ("split_k", 2, 2)),   # more rows: the earlier rules
])
def test_double_small_rows(sa, sb, want):
    """DOUBLE over at most 32 rows runs on the 32 x 128 entry, splitting K
    up to one tile per CU."""
    inf = mm.Plan(sa, sb, mm.DOUBLE).info()
    assert (mm.ALGO_NAMES[inf["algo"]], inf["tile"], inf["split_k"]) == want, inf


# ---------------------------------------------------------------- last-round balancing

def test_tail_split_plans():
    """A large tile that leaves the last round of workgroups less than half
    full covers the leading columns in whole rounds and hands the rest to a
    second launch; shapes whose tiles fill whole rounds, forced tiles and
    DOUBLE keep one launch."""
    p = mm.Plan((16, 512, 4096), (4096, 11008), mm.BFLOAT16)
    inf = p.info()
    assert inf["tile"] == 1 and inf["tail_col"] == 10240 and inf["tail_tile"] >= 1
    bm, bn, _ = mm.tile_configs(mm.BFLOAT16)[inf["tile"] - 1]
    tiles_main = (inf["kernel_m"] // bm) * (inf["tail_col"] // bn)
    assert tiles_main % 256 == 0  # whole rounds on 256 CUs
    for sa, sb, dt in [((4, 32, 2048, 128), (4, 32, 128, 2048), mm.BFLOAT16),
                       ((8192, 8192), (8192, 8192), mm.BFLOAT16),
                       ((1024, 1024), (1024, 1024), mm.FLOAT),
                       ((16, 512, 4096), (4096, 11008), mm.DOUBLE)]:
        assert mm.Plan(sa, sb, dt).info()["tail_col"] == 0
    forced = mm.Plan((16, 512, 4096), (4096, 11008), mm.BFLOAT16, force_algo=mm.ALGO_GENERAL, tile=1)
    assert forced.info()["tail_col"] == 0


# 16-bit entry 10 (tile 11) is the persistent twin of the 256 x 256 entry.
PERSIST_TILE = 11


@pytest.mark.parametrize("sa,sb,dt,tile", [
    ((4, 32, 2048, 128), (4, 32, 128, 2048), mm.BFLOAT16, PERSIST_TILE),  # QK^T: K = 128, 32 rounds
    ((8192, 1024), (1024, 8192), mm.FLOAT16, PERSIST_TILE),               # K = 1024, 4 rounds
    ((8192, 2048), (2048, 8192), mm.BFLOAT16, 1),                         # K = 2048: the plain kernel
    ((16, 512, 4096), (4096, 11008), mm.BFLOAT16, 1),                      # long K (and a column split)
    ((4, 32, 2000, 128), (4, 32, 128, 2048), mm.BFLOAT16, 1),             # rows not whole tiles
    ((4, 32, 2048, 120), (4, 32, 120, 2048), mm.BFLOAT16, 1),             # K not whole stages
    ((2048, 128), (128, 2048), mm.BFLOAT16, None),                        # 64 tiles: under two rounds
])
def test_persistent_selection(sa, sb, dt, tile):
    """Short-K 16-bit products of whole 256 x 256 tiles and stages, with at
    least two rounds of tiles, run the persistent kernel."""
    assert mm.tile_configs(dt)[PERSIST_TILE - 1] == mm.tile_configs(dt)[0]
    inf = mm.Plan(sa, sb, dt).info()
    assert mm.ALGO_NAMES[inf["algo"]] == "general"
    assert inf["tile"] == tile if tile is not None else inf["tile"] != PERSIST_TILE


@pytest.mark.parametrize("M,K,N,want", [
    (16, 4096, 4096, ("split_k", 14, 8)),     # 32 tiles of 64 x 128: 8 chunks, at most 2 per CU
    (32, 4096, 11008, ("split_k", 14, 4)),    # 86 tiles: 4 chunks
    (16, 4096, 12288, ("split_k", 14, 4)),
    (64, 14336, 4096, ("split_k", 14, 8)),    # chunks capped at 8
    (16, 2048, 8192, ("split_k", 14, 4)),     # chunks at least 512 long
    (16, 4096, 2048, ("split_k", 5, 8)),      # 16 tiles x 8 chunks leave CUs idle: the earlier rule
    (16, 1024, 4096, ("split_k", 5, 4)),
    (16, 4096, 28672, ("general", 5, 1)),     # more than half a round of tiles
    (65, 4096, 4096, None),                   # more rows
])
def test_gemm_linear_split(M, K, N, want):
    """A 16-bit Gemm with B transposed (a linear layer) over at most 64 rows
    splits K on the 64 x 128 entry, in the largest power-of-two chunk count
    with at most two workgroups per CU (capped at K / 512 and 8), when
    the chunks give every CU a workgroup."""
    for dt in (mm.BFLOAT16, mm.FLOAT16):
        inf = mm.GemmPlan((M, K), (N, K), dt, False, True, (N,), 1.0, 1.0).info()
        got = (mm.ALGO_NAMES[inf["algo"]], inf["tile"], inf["split_k"])
        if want is None:
            assert got[1] != 14, got
        else:
            assert got == want, (M, K, N, got)
    # B not transposed, A transposed, or FP32: the rule does not apply
    assert mm.GemmPlan((16, 4096), (4096, 4096), mm.BFLOAT16, False, False).info()["tile"] != 14
    assert mm.GemmPlan((4096, 16), (4096, 4096), mm.BFLOAT16, True, True).info()["tile"] != 14
    assert mm.GemmPlan((16, 4096), (4096, 4096), mm.FLOAT, False, True).info()["tile"] != 14


@pytest.mark.parametrize("M,K,N,want", [
    (16, 4096, 4096, ("split_k", 8, 8)),      # 32 tiles of 32 x 128: 8 chunks, one workgroup per CU
    (32, 4096, 11008, ("split_k", 8, 2)),     # 86 tiles: 2 chunks, not 3 (258 workgroups)
    (16, 8192, 8192, ("split_k", 8, 4)),
    (16, 2048, 2048, ("split_k", 8, 8)),      # 16 tiles: at most K / 256 chunks
    (16, 1024, 4096, ("split_k", 8, 4)),
    (16, 4096, 28672, ("split_k", 8, 2)),     # up to one tile per CU: at least 2 chunks
    (32, 4096, 40000, ("general", 8, 1)),     # past one tile per CU
])
def test_float_small_rows(M, K, N, want):
    """FP32 MatMul (where skinny-M does not take it) and Gemm of at most 32
    rows run on the 32 x 128 entry with two K groups, splitting K up to one
    tile per CU."""
    assert mm.tile_configs(mm.FLOAT)[7] == (32, 128, 32)
    inf = mm.Plan((M, K), (K, N), mm.FLOAT).info()
    assert (mm.ALGO_NAMES[inf["algo"]], inf["tile"], inf["split_k"]) == want, inf
    for ta, tb in ((0, 0), (0, 1), (1, 0), (1, 1)):
        sa = (K, M) if ta else (M, K)
        sb = (N, K) if tb else (K, N)
        g = mm.GemmPlan(sa, sb, mm.FLOAT, ta, tb, (N,), 1.0, 1.0).info()
        assert (mm.ALGO_NAMES[g["algo"]], g["tile"], g["split_k"]) == want, (ta, tb, g)
    # more rows keep the other rules; few-row MatMul keeps skinny-M where it wins
    assert mm.Plan((33, 4096), (4096, 11008), mm.FLOAT).info()["tile"] != 8
    assert mm.Plan((8, 4096), (4096, 8704), mm.FLOAT).algo == mm.ALGO_SKINNY_M
    assert mm.Plan((15, 4096), (4096, 8704), mm.FLOAT).info()["tile"] == 8


@pytest.mark.parametrize("sa,sb,want", [
    ((128, 4096), (4096, 11008), ("split_k", 6, 2)),   # 2 chunks of 64 x 64, not 3 of 128 x 128 (258 workgroups)
    ((256, 2048), (2048, 2048), ("split_k", 6, 2)),
    ((512, 11008), (11008, 4096), ("split_k", 7, 4)),
    ((128, 8192), (8192, 8192), ("split_k", 7, 4)),
    ((512, 2048), (2048, 2048), ("general", 6, 1)),    # a 1 % estimated gain does not pay the reduction
    ((512, 8192), (8192, 8192), ("split_k", 7, 2)),
    ((1024, 8192), (8192, 8192), ("general", 7, 1)),   # more rows: the earlier rules
    ((64, 131072), (131072, 64), ("split_k", 6, 256)),  # one tile: 256 chunks of 512
])
def test_float_timed_split(sa, sb, want):
    """FP32 products of 33-512 rows split K when the time model's estimate
    of the chunks, their partials and the reduction beats the general
    plan's."""
    inf = mm.Plan(sa, sb, mm.FLOAT).info()
    assert (mm.ALGO_NAMES[inf["algo"]], inf["tile"], inf["split_k"]) == want, inf


# ---------------------------------------------------------------- constant B

def test_constant_b_errors_before_any_gpu_call():
    """The constant-B storage must hold exactly the planned matrix, and the
    B-less execute is refused while the plan owns no B (both checked before
    any device call)."""
    L = mm.lib()
    p = mm.Plan((4, 64, 96), (96, 80), mm.FLOAT)
    assert not p.has_constant_b
    with pytest.raises(mm.MMError) as e:
        p.execute_constant_b_ptr(0, 0)
    assert e.value.status == mm.ERR_NO_CONSTANT_B
    for numel in (96 * 80 - 1, 96 * 80 + 1, 0):
        with pytest.raises(mm.MMError) as e:
            p.set_constant_b_ptr(0, numel)
        assert e.value.status == mm.ERR_SIZE
    assert L.mm_plan_set_constant_b(None, None, 0, None) == mm.ERR_NULL_ARG
    assert L.mm_plan_has_constant_b(None) == 0
    assert L.mm_execute_constant_b(None, None, None, None) == mm.ERR_NULL_ARG
    assert not p.has_constant_b
    # constant B serves mm_execute only: Gemm and MatMulInteger plans refuse it
    for q in (mm.GemmPlan((64, 96), (96, 80), mm.FLOAT), mm.IntPlan((64, 96), (96, 80), mm.UINT8, mm.INT8)):
        with pytest.raises(mm.MMError) as e:
            q.set_constant_b_ptr(0, 96 * 80)
        assert e.value.status == mm.ERR_BAD_OPTION and not q.has_constant_b


# ---------------------------------------------------------------- Gemm

@pytest.mark.parametrize("ta,tb", [(0, 0), (1, 0), (0, 1), (1, 1)])
def test_gemm_plan_shapes(ta, tb):
    M, N, K = 300, 200, 520
    sa = (K, M) if ta else (M, K)
    sb = (N, K) if tb else (K, N)
    p = mm.GemmPlan(sa, sb, mm.BFLOAT16, trans_a=ta, trans_b=tb, c_shape=(N,), alpha=0.5, beta=2.0)
    assert p.output_shape == (M, N) and p.output_numel == M * N
    inf = p.info()
    assert (inf["M"], inf["N"], inf["K"]) == (M, N, K) and inf["algo"] == mm.ALGO_GENERAL
    assert inf["tile"] - 1 in (0, 5, 4, 2, 1, 13)  # Gemm: only the tiles instantiated with its epilogue
    assert inf["tail_col"] == 0
    # skinny shapes of a Gemm take the tiled kernels: split-K when one row
    # of tiles cannot fill the GPU and K is long, else the general kernel
    assert mm.GemmPlan((1, 4096), (4096, 4096), mm.FLOAT16).algo == mm.ALGO_SPLIT_K
    assert mm.GemmPlan((1, 512), (512, 4096), mm.FLOAT16).algo == mm.ALGO_GENERAL
    assert mm.GemmPlan((4096, 64), (64, 0), mm.FLOAT16).algo == mm.ALGO_EMPTY
    assert mm.GemmPlan((64, 0), (0, 32), mm.FLOAT16, c_shape=(1,)).algo == mm.ALGO_DIRECT  # Y = beta * C


@pytest.mark.parametrize("kw,status", [
    (dict(sa=(4, 3), sb=(4, 5)), mm.ERR_K_MISMATCH),
    (dict(sa=(4, 3), sb=(3, 5), c_shape=(4, 2)), mm.ERR_BROADCAST),
    (dict(sa=(4, 3), sb=(3, 5), c_shape=(4,)), mm.ERR_BROADCAST),
    (dict(sa=(4, 3), sb=(3, 5), c_shape=(5, 4)), mm.ERR_BROADCAST),
    (dict(sa=(4, -3), sb=(3, 5)), mm.ERR_NEG_DIM),
    (dict(sa=(4, 3), sb=(3, 5), c_shape=(-1,)), mm.ERR_NEG_DIM),
    (dict(sa=(4, 3), sb=(3, 5), dtype=mm.DOUBLE), mm.ERR_DTYPE),
    (dict(sa=(64, 64), sb=(64, 8), force_algo=mm.ALGO_SKINNY_N), mm.ERR_BAD_OPTION),
    (dict(sa=(64, 64), sb=(64, 64), trans_a=1, force_algo=mm.ALGO_GENERAL, tile=4), mm.ERR_BAD_OPTION),
])
def test_gemm_plan_errors(kw, status):
    kw = dict(kw)
    sa, sb = kw.pop("sa"), kw.pop("sb")
    dt = kw.pop("dtype", mm.FLOAT16)
    with pytest.raises(mm.MMError) as e:
        mm.GemmPlan(sa, sb, dt, **kw)
    assert e.value.status == status


def test_gemm_execute_checks_before_any_gpu_call():
    """A Gemm plan is refused by mm_execute and a MatMul plan by
    mm_gemm_execute; a plan with C refuses a NULL C."""
    L = mm.lib()
    g = mm.GemmPlan((64, 32), (32, 16), mm.FLOAT, c_shape=(1, 16))
    m = mm.Plan((64, 32), (32, 16), mm.FLOAT)
    fake = ctypes.c_void_p(1 << 40)
    assert L.mm_execute(g.handle, fake, fake, fake, None) == mm.ERR_BAD_OPTION
    assert L.mm_gemm_execute(m.handle, fake, fake, None, fake, None) == mm.ERR_BAD_OPTION
    assert L.mm_gemm_execute(g.handle, fake, fake, None, fake, None) == mm.ERR_NULL_ARG


# ---------------------------------------------------------------- MatMulInteger

@pytest.mark.parametrize("ta,tb,zka,zkb,ra,cb", [
    (mm.INT8, mm.INT8, mm.ZP_NONE, mm.ZP_NONE, False, False),
    (mm.UINT8, mm.INT8, mm.ZP_NONE, mm.ZP_NONE, False, True),
    (mm.INT8, mm.UINT8, mm.ZP_NONE, mm.ZP_NONE, True, False),
    (mm.INT8, mm.INT8, mm.ZP_SCALAR, mm.ZP_NONE, False, True),
    (mm.INT8, mm.INT8, mm.ZP_NONE, mm.ZP_VECTOR, True, False),
    (mm.UINT8, mm.UINT8, mm.ZP_VECTOR, mm.ZP_SCALAR, True, True),
])
def test_int_plan_shapes(ta, tb, zka, zkb, ra, cb):
    """Every signedness / zero-point combination plans the tiled kernel with
    no workspace (the kernel forms the row and column sums it needs)."""
    p = mm.IntPlan((4, 1, 64, 128), (3, 128, 96), ta, tb, zka, zkb)
    assert p.output_shape == (4, 3, 64, 96)
    inf = p.info()
    assert inf["dtype"] == mm.INT32 and inf["algo"] == mm.ALGO_GENERAL and not inf["folded"]
    assert inf["min_bytes"] == 4 * 64 * 128 + 3 * 128 * 96 + 4 * 4 * 3 * 64 * 96
    assert p.workspace_bytes == 0


def test_int_plan_algorithms():
    u8, s8 = mm.UINT8, mm.INT8
    f = mm.IntPlan((8, 64, 256), (256, 128), u8, s8)
    assert f.info()["folded"] and f.info()["kernel_m"] == 512 and f.algo == mm.ALGO_GENERAL
    assert f.workspace_bytes == 0
    # no skinny kernels: few tiles over a long K split K (INT32 partials)
    assert mm.IntPlan((1, 4096), (4096, 4096), s8, s8).algo == mm.ALGO_SPLIT_K
    assert mm.IntPlan((4096, 4096), (4096, 1), s8, s8).algo == mm.ALGO_GENERAL
    assert mm.IntPlan((8, 16), (16, 8), s8, s8).algo == mm.ALGO_DIRECT
    assert mm.IntPlan((64, 0), (0, 32), s8, u8).algo == mm.ALGO_ZERO_FILL
    assert mm.IntPlan((0, 64), (64, 32), s8, u8).algo == mm.ALGO_EMPTY
    d = mm.IntPlan((512, 512), (512, 512), u8, u8, force_algo=mm.ALGO_DIRECT)
    assert d.algo == mm.ALGO_DIRECT and d.workspace_bytes == 0
    t = mm.IntPlan((512, 512), (512, 512), u8, u8, force_algo=mm.ALGO_GENERAL, tile=2)
    assert t.info()["tile"] == 2
    assert mm.tile_configs(mm.INT8) == mm.tile_configs(mm.UINT8) == [(256, 256, 128), (128, 128, 128), (256, 256, 128),
                                                                      (64, 128, 128), (128, 128, 128)]
    # the 256 x 256 entry whose waves hold fewer fragments of a sign-flipped A
    assert mm.IntPlan((4096, 4096), (4096, 4096), u8, s8).info()["tile"] == 3
    assert mm.IntPlan((4096, 4096), (4096, 4096), s8, u8).info()["tile"] == 1
    assert mm.IntPlan((4096, 4096), (4096, 4096), u8, u8).info()["tile"] == 1
    assert mm.tile_configs(mm.INT32) == mm.tile_configs(mm.INT8)


@pytest.mark.parametrize("kw,status", [
    (dict(ta=mm.FLOAT), mm.ERR_DTYPE),
    (dict(tb=mm.INT32), mm.ERR_DTYPE),
    (dict(zka=3), mm.ERR_BAD_OPTION),
    (dict(zkb=-1), mm.ERR_BAD_OPTION),
    (dict(force_algo=mm.ALGO_SKINNY_M), mm.ERR_BAD_OPTION),
    (dict(force_algo=mm.ALGO_SPLIT_K, tile=1), mm.ERR_BAD_OPTION),  # split-K: the 128 x 128 entry only
    (dict(force_algo=mm.ALGO_GENERAL, tile=6), mm.ERR_BAD_OPTION),
    (dict(sb=(100, 64)), mm.ERR_K_MISMATCH),
    (dict(sa=(3, 64, 128), sb=(2, 128, 64)), mm.ERR_BROADCAST),
])
def test_int_plan_errors(kw, status):
    kw = dict(kw)
    sa, sb = kw.pop("sa", (64, 128)), kw.pop("sb", (128, 64))
    args = (kw.pop("ta", mm.INT8), kw.pop("tb", mm.UINT8), kw.pop("zka", 0), kw.pop("zkb", 0))
    with pytest.raises(mm.MMError) as e:
        mm.IntPlan(sa, sb, *args, **kw)
    assert e.value.status == status


@pytest.mark.parametrize("sa,sb,want", [
    ((16, 4096), (4096, 11008), ("split_k", 4, 3)),   # 86 tiles of 64 x 128 (three stages): 3 chunks
    ((16, 11008), (11008, 4096), ("split_k", 4, 8)),
    ((2, 8, 4096), (2, 4096, 2048), ("split_k", 4, 8)),  # batched: 2 x 16 tiles
    ((96, 4096), (4096, 4096), ("split_k", 5, 8)),    # more rows, 32 tiles x 8 chunks fill the CUs: three stages
    ((128, 4096), (4096, 11008), ("split_k", 2, 3)),  # 86 tiles x 3 chunks overflow them: two-stage 128 x 128
    ((64, 4096), (4096, 28672), ("general", 4, 1)),   # 224 tiles: no split, the 64 x 128 entry whole
    ((16, 4096), (4096, 65536), ("general", 2, 1)),   # past one round of 128-column tiles: 128 x 128
    ((16, 4100), (4100, 4096), ("general", 4, 1)),    # K not whole 16-byte chunks: no split (the tiled kernel's limit)
    ((16, 512, 4096), (4096, 11008), ("general", 3, 1)),
])
def test_int_split_plans(sa, sb, want):
    """MatMulInteger splits K where the other types' rules split (few tiles,
    long K) and the tiled kernel takes the shape, on the three-stage 64 x 128
    entry up to 64 rows and the 128 x 128 one beyond, with INT32 partials in
    a workspace of split x rows x N x 4 bytes."""
    p = mm.IntPlan(sa, sb, mm.UINT8, mm.INT8, mm.ZP_SCALAR, mm.ZP_VECTOR)
    inf = p.info()
    assert (mm.ALGO_NAMES[inf["algo"]], inf["tile"], inf["split_k"]) == want, inf
    if want[0] == "split_k":
        assert inf["k_chunk"] % 128 == 0  # partitions hold whole 128-byte stages
        assert p.workspace_bytes == inf["split_k"] * inf["batch"] * inf["kernel_m"] * inf["N"] * 4
    f = mm.IntPlan((16, 1000), (1000, 256), mm.INT8, mm.INT8, force_algo=mm.ALGO_SPLIT_K, split_k=3)
    assert (f.algo, f.info()["tile"], f.info()["split_k"]) == (mm.ALGO_SPLIT_K, 4, 3)


def test_int_execute_checks_before_any_gpu_call():
    """A MatMulInteger plan is refused by mm_execute and a MatMul plan by
    mm_int_execute; a plan with zero points refuses NULL zero points."""
    L = mm.lib()
    q = mm.IntPlan((64, 256), (256, 128), mm.UINT8, mm.INT8, mm.ZP_SCALAR, mm.ZP_VECTOR)
    m = mm.Plan((64, 32), (32, 16), mm.FLOAT)
    fake = ctypes.c_void_p(1 << 40)
    assert L.mm_execute(q.handle, fake, fake, fake, None) == mm.ERR_BAD_OPTION
    assert L.mm_int_execute(m.handle, fake, fake, None, None, fake, None) == mm.ERR_BAD_OPTION
    assert L.mm_int_execute(q.handle, fake, fake, None, fake, fake, None) == mm.ERR_NULL_ARG
    assert L.mm_int_execute(q.handle, fake, fake, fake, None, fake, None) == mm.ERR_NULL_ARG
    assert L.mm_int_execute(q.handle, None, fake, fake, fake, fake, None) == mm.ERR_NULL_ARG
    assert L.mm_int_execute(None, fake, fake, fake, fake, fake, None) == mm.ERR_NULL_ARG
    assert L.mm_int_plan_create(None, 2, None, 2, mm.INT8, mm.INT8, 0, 0, None, None) == mm.ERR_NULL_ARG
