"""The bench's measurement model on the CPU: the algorithmic bytes it divides
by (per kernel, at 8192 x 8192) and the access-shape codes it launches, which
must be the ones include/mxq_shapes.h declares."""
import importlib.util
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_model", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_algorithmic_bytes_at_8192():
    """n = 8192^2 elements, B = n / 32 blocks, T = n / 16384 tiles: the byte
    model of each step kernel, bf16 and fp32."""
    b = _bench()
    n = 8192 * 8192
    B, T = n // 32, n // 16384
    assert b.algorithmic_bytes(8192, 8192, 2) == {
        "proj": 4 * n, "row": 2 * n + n + B, "export": 2 * B, "block128": 2 * n + n + T,
        "dec_row": n + B + 2 * n, "dec_tile": n + T + 2 * n}
    a4 = b.algorithmic_bytes(8192, 8192, 4)
    assert a4["proj"] == 8 * n and a4["row"] == 4 * n + n + B and a4["dec_tile"] == n + T + 4 * n
    assert b.algorithmic_bytes(8192, 8192, 2)["row"] == 203_423_744
    assert b.algorithmic_bytes(8192, 8192, 2)["block128"] == 201_330_688
    assert sum(b.algorithmic_bytes(8192, 8192, 2).values()) == 1_082_138_624


def test_widened_kernel_bytes():
    b = _bench()
    n = 8192 * 8192
    B, T = n // 32, n // 16384
    assert b.packed_bytes(8192, 8192, 2) == {"quantize_mxfp4": 2 * n + n // 2 + B, "dequantize_mxfp4": n // 2 + B + 2 * n,
                                             "packed_to_row": n // 2 + B + n + B, "packed_to_block128": n // 2 + B + n + T}
    assert b.fused_bytes(8192, 8192, 2) == 2 * n + 2 * n + n + B
    nc = (8192 // 32) * 8192
    assert b.col_bytes(8192, 8192, 2) == {"col": 2 * n + n + nc, "row_col": 2 * n + n + B + n + nc,
                                          "dec_col": n + nc + 2 * n}


def test_ragged_shapes_round_blocks_and_tiles_up():
    b = _bench()
    a = b.algorithmic_bytes(100, 48, 2)
    assert a["row"] == 2 * 4800 + 4800 + 100 * 2 and a["block128"] == 2 * 4800 + 4800 + 1


def test_access_shape_codes_match_the_header():
    b = _bench()
    text = open(os.path.join(ROOT, "include", "mxq_shapes.h")).read()
    enum = {m.group(1): int(m.group(2)) for m in re.finditer(r"MXQ_SHAPE_(\w+)\s*=\s*(\d+)", text)}
    assert len(enum) == len(b.SHAPES_OF)
    for name, (code, _, _) in b.SHAPES_OF.items():
        assert enum[name[len("shape_"):].upper()] == code, name
    assert set(b.SHAPE_KERNEL) <= set(b.SHAPES_OF)
