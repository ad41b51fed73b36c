"""Host-side logic of bench.py (no GPU): kernel choice per shape and variant,
algorithmic byte counts, the single-GPU refusal, and the profile digests."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_kernel_family():
    assert bench.kernel_family(8, 4096) == "decode"
    assert bench.kernel_family(16, 4096) == "fused"
    assert bench.kernel_family(16, 8192) == "small_m"
    assert bench.kernel_family(2048, 4096) == "tiled"
    # up to 64 rows, the weight-streaming kernel while M * N * K <= 6e9 or
    # its grid is one round of the chip
    assert bench.kernel_family(17, 8192, N=28672) == "small_m"
    assert bench.kernel_family(32, 8192, N=28672) == "small_m"
    assert bench.kernel_family(32, 8192, N=57344) == "tiled"
    assert bench.kernel_family(48, 8192, N=28672) == "tiled"
    assert bench.kernel_family(64, 4096, N=16384) == "small_m"
    assert bench.kernel_family(64, 16384, N=16384) == "small_m"
    assert bench.kernel_family(32, 28672, N=8192) == "small_m"
    assert bench.kernel_family(64, 8192, N=20480) == "tiled"
    assert bench.kernel_family(64, 28672, N=8192) == "tiled"
    assert bench.kernel_family(65, 4096, N=1024) == "tiled"
    # the FP8 forward has the fused decode kernel, not the other fused one
    assert bench.kernel_family(8, 4096, "fp8") == "decode"
    assert bench.kernel_family(16, 4096, "fp8") == "small_m"
    assert bench.kernel_family(2048, 4096, "fp8") == "tiled"


def test_algorithmic_bytes_decode():
    M, N, K, n_out = 8, 4096, 4096, 4
    b = bench.algorithmic_bytes("decode", M, N, K, n_out, False)
    # int8 weight + its scales + fp16 X in + Y out + the activation outputs
    assert b == N * K + 4 * N + 2 * M * N + 2 * M * K + M * K + 4 * M + 2 * M * 32 + 4 * n_out + 4


def test_refuses_several_gpus():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert p.returncode == 2 and "one GPU" in p.stderr


def test_profile_digests_name_their_kernel_sources():
    prof = os.path.join(ROOT, "profiles")
    for name in sorted(os.listdir(prof)):
        if name.startswith("traffic_") and name.endswith(".json"):
            with open(os.path.join(prof, name)) as f:
                t = json.load(f)
            assert t["kernel"] in bench.KERNEL_NAMES.values(), name
            assert t["hbm_bytes_per_launch"] > 0 and t["algorithmic_bytes_per_launch"] > 0


def test_small_m_rule_matches_library():
    """bench.py's kernel family follows the library's choice of the streaming
    product: its workspace size is 0 exactly for those shapes (M > 16)."""
    import int8_quantized_matmul_row_amd as pkg
    for M in (17, 32, 33, 48, 64, 65, 100):
        for N, K in ((4096, 4096), (16384, 4096), (28672, 8192), (57344, 14336), (700, 2048),
                     (16384, 16384), (16400, 16384), (8192, 28672), (8208, 28672), (20480, 8192)):
            streaming = pkg.llmint8_matmul_workspace_size(M, N, K) == 0
            assert streaming == bench.small_m_product(M, N, K), (M, N, K)
