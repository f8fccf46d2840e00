"""Host-side logic of bench.py and of the binding's prepared calls (no GPU)."""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import datagen  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_algorithmic_bytes_q_proj():
    """Quantize: X bf16 read once, codes and scales written; GEMM: codes and scales of both
    operands read once, Y bf16 written (the sizes of the q_proj configuration)."""
    wl = datagen.make("q_proj", M=2048, K=4096, N=4096)
    q, g = bench.algorithmic_bytes(wl)
    assert q == 2048 * 4096 * 2 + 2048 * 2048 + 2048 * 32 * 4 == 21233664
    assert g == 2048 * 2048 + 2048 * 32 * 4 + 4096 * 2048 + 4096 * 32 * 4 + 2048 * 4096 * 2 == 30146560
    q64, g64 = bench.algorithmic_bytes(wl, 64)
    assert q64 - q == 2048 * 32 * 4 and g64 - g == (2048 + 4096) * 32 * 4


@pytest.mark.parametrize("M,N,kernel", [
    (1, 4096, "gemm_small_kernel"), (64, 14336, "gemm_small_kernel"),
    (65, 4096, "gemm_small_kernel"), (384, 4096, "gemm_small_kernel"),   # 3 x 32 tiles < 128
    (512, 4096, "gemm_f8p_kernel"),                                      # 4 x 32 tiles
    (128, 14336, "gemm_small_kernel"), (256, 14336, "gemm_f8p_kernel"),
    (1024, 40, "gemm_small_kernel"), (1025, 40, "gemm_f8p_kernel"),
    (2048, 4096, "gemm_f8p_kernel"),
])
def test_gemm_routing(M, N, kernel):
    assert bench.gemm_kernel_for(M, N) == kernel
    # 64- and 256-wide groups keep the unpipelined tiled kernel
    assert bench.gemm_kernel_for(M, N, 256) == kernel.replace("f8p", "f8")


def test_traffic_lookup():
    assert bench.measured_traffic("gemm_f8_kernel", "no_such_workload") is None
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as fh:
        table = json.load(fh)
    for key, rec in table.items():
        kernel, _, workload = key.partition(":")
        assert kernel in bench.KERNEL_SOURCES, key
        assert rec["hbm_bytes_per_launch"] > 0 and rec["algorithmic_bytes"] > 0
        got = bench.measured_traffic(kernel, workload)
        # a record counts only while the kernel's sources are the ones it was measured on
        assert got == (rec["hbm_bytes_per_launch"] if rec["source_hash"] == bench.kernel_source_hash(kernel) else None)


def test_prepared_calls_refuse_host_tensors():
    torch = pytest.importorskip("torch")
    rw4 = pytest.importorskip("rotated_w4a4_amd")
    K, M, N = 256, 4, 8
    qa = torch.zeros((M, K // 2), dtype=torch.uint8)
    sa = torch.zeros((M, K // 128), dtype=torch.float32)
    qw = torch.zeros((N, K // 2), dtype=torch.uint8)
    sw = torch.zeros((N, K // 128), dtype=torch.float32)
    with pytest.raises(ValueError, match="GPU"):
        rw4.prepare_w4a4_gemm(qa, sa, qw, sw, torch.float32)
    with pytest.raises(ValueError, match="GPU"):
        rw4.prepare_dequantize(qa, sa, torch.float32)
    t = rw4.Transform.__new__(rw4.Transform)  # no device tables are needed to reach the checks
    t._h, t.K, t.kind = None, K, "hadamard128"
    with pytest.raises(ValueError, match="GPU"):
        rw4.prepare_quantize_act(t, torch.zeros((M, K), dtype=torch.bfloat16))
    assert np.all(qa.numpy() == 0)  # nothing was written


def test_algorithmic_bytes_givens_counts_the_lookup_table():
    """The decode quantizer also reads the Givens table: 2-byte pair index and 8-byte
    (cos, sin) per (group, layer, slot) and alpha^-1 per channel = 176 KiB at K = 4096,
    8 layers; M = 16 gives 16 * (8192 + 2048 + 128) + 180224 = 346112 bytes."""
    wl = datagen.make("decode", M=16)
    q, _ = bench.algorithmic_bytes(wl)
    assert bench.givens_table_bytes(4096, 8) == 176 * 1024
    assert q == 346112


def test_spread_reports_median_and_percentiles():
    s = bench.spread([5.0, 1.0, 3.0, 2.0, 4.0])
    assert s["median"] == 3.0 and s["n"] == 5
    assert s["p10"] == pytest.approx(1.4) and s["p90"] == pytest.approx(4.6)
