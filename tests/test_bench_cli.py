"""Host-side parts of bench.py: the command-line product specs (no GPU)."""
import pytest

import bench
from onnx_broadcast_matmul_amd import binding as mm
from onnx_broadcast_matmul_amd import synth


def test_parse_shapes():
    p = bench.parse_shapes("bf16:16x4096/4096x65536,fp32:linear:16x4096x11008,fp16:2x16x2048/2x2048x4096")
    assert isinstance(p[0], synth.Product) and p[0].a_shape == (16, 4096) and p[0].b_shape == (4096, 65536)
    assert p[0].dtype == mm.BFLOAT16 and p[0].name == "bf16_16x4096_by_4096x65536"
    g = p[1]
    assert isinstance(g, synth.GemmProduct) and (g.M, g.K, g.N) == (16, 4096, 11008)
    assert g.trans_b and not g.trans_a and g.c_shape == (11008,) and g.dtype == mm.FLOAT
    assert p[2].a_shape == (2, 16, 2048) and p[2].dtype == mm.FLOAT16
    (q,) = bench.parse_shapes("u8s8:16x4096/4096x11008")
    assert isinstance(q, synth.IntProduct) and q.a_shape == (16, 4096) and not q.a_signed and q.b_signed
    assert q.a_zp == 0 and q.b_zp == 0


@pytest.mark.parametrize("bad", ["int8:4x4/4x4", "bf16", "bf16:4x4"])
def test_parse_shapes_rejects(bad):
    with pytest.raises(ValueError):
        bench.parse_shapes(bad)
