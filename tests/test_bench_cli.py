"""bench.py's command-line contract, checked without a GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120)


def test_more_than_one_gpu_exits_with_a_message():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_step_count_must_be_positive():
    r = _run("--steps", "0")
    assert r.returncode != 0 and "--steps" in r.stderr


def test_algorithmic_bytes_at_8192():
    sys.path.insert(0, ROOT)
    import bench
    b = bench.algorithmic_bytes(8192, 8192)
    assert b["proj"] == 268435456 and b["row"] == 203423744 and b["block128"] == 201330688
    assert bench.fused_bytes(8192, 8192) == 337641472
    assert bench.col_bytes(8192, 8192)["col"] == 203423744


def test_algorithmic_bytes_fp32_weight():
    """The fp32 master weight: 4-byte elements in, and the decodes write fp32."""
    sys.path.insert(0, ROOT)
    import bench
    n, nb = 8192 * 8192, 8192 * 256
    b = bench.algorithmic_bytes(8192, 8192, 4)
    assert b["proj"] == 8 * n and b["row"] == 4 * n + n + nb and b["dec_row"] == n + nb + 4 * n
    assert b["export"] == bench.algorithmic_bytes(8192, 8192)["export"]
    assert bench.fused_bytes(8192, 8192, 4) == 9 * n + nb
    assert bench.packed_bytes(8192, 8192, 4)["dequantize_mxfp4"] == n // 2 + nb + 4 * n


def test_weight_choice_is_validated():
    r = _run("--weight", "fp16")
    assert r.returncode != 0 and "--weight" in r.stderr


def test_algorithmic_bytes_mlp_shapes():
    """The MLP-shaped weights: 28672 x 8192 bf16 and its fp32 master (the byte
    model at n = 28672 * 8192 elements and n / 32 blocks)."""
    sys.path.insert(0, ROOT)
    import bench
    b = bench.algorithmic_bytes(28672, 8192)
    assert b["proj"] == 939524096 and b["row"] == 711983104
    b = bench.algorithmic_bytes(28672, 8192, 4)
    assert b["proj"] == 1879048192 and b["row"] == 1181745152
    # the transposed weight moves the same bytes except where blocks and tiles are counted
    assert bench.algorithmic_bytes(8192, 28672)["proj"] == 939524096
    assert bench.algorithmic_bytes(8192, 28672)["export"] == 2 * 8192 * 896


def test_shape_choice_is_validated():
    r = _run("--shape", "100x48")
    assert r.returncode != 0 and "--shape" in r.stderr
    r = _run("--shape", "8192x28672", "--weight", "fp32")
    assert r.returncode == 2 and "fp32 master" in r.stderr
