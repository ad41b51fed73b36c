"""Per-tensor absmax quantization (the baseline scheme) on the GPU against the
oracle: codes and scale bit-exact, and its int8 product through llmint8_matmul
with no outliers.

"A Gentle Introduction to 8-bit Matrix Multiplication for transformers at
scale", section "absmax quantization"."""
import numpy as np
import pytest

import synth
from gpu_helpers import bits_of, check_y, log, to_torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


CASES = [(1, 64, synth.F16), (37, 320, synth.BF16), (300, 1024, synth.F16),
         (2048, 4096, synth.BF16)]


@pytest.mark.parametrize("R,C,dt", CASES, ids=[f"{r}x{c}-{synth.DTYPE_NAMES[d]}" for r, c, d in CASES])
def test_quantize_tensor_bit_exact(orc, R, C, dt):
    import torch
    import int8_quantized_matmul_row_amd as pkg
    wl = synth.make_random(R, 1, C, dt, seed=R + C, n_outlier_cols=2)
    A = wl.X.copy()
    a = synth.bits_to_f32(A, dt)
    a[R - 1, C - 1] = -3.0 * np.abs(a).max()   # the absmax in the very last element
    A = synth.to_bits(a, dt)
    log(f"[per-tensor] {R}x{C}")
    Q, scale = pkg.quantize_tensor(to_torch(A, dt, "cuda"))
    torch.cuda.synchronize()
    Qr, sr = orc.quantize_tensor(A, dt)
    assert np.array_equal(Q.cpu().numpy(), Qr)
    assert np.array_equal(scale.cpu().numpy(), sr)


def test_quantize_tensor_all_zero():
    import torch
    import int8_quantized_matmul_row_amd as pkg
    A = torch.zeros((5, 128), dtype=torch.float16, device="cuda")
    Q, scale = pkg.quantize_tensor(A)
    torch.cuda.synchronize()
    assert not Q.any().item() and not scale.any().item()


@pytest.mark.parametrize("M,N,K,dt", [(8, 300, 512, synth.F16), (96, 520, 640, synth.BF16)])
def test_per_tensor_product_matches_oracle(orc, M, N, K, dt):
    import torch
    import int8_quantized_matmul_row_amd as pkg
    wl = synth.make_random(M, N, K, dt, seed=5 + M, n_outlier_cols=3, bias_sigma=0.01)
    X, W = to_torch(wl.X, dt, "cuda"), to_torch(wl.W, dt, "cuda")
    bias = to_torch(wl.bias, dt, "cuda")
    Qx, sx = pkg.quantize_tensor(X)
    Qw, sw = pkg.quantize_tensor(W)
    Y = pkg.matmul_codes(Qx, sx, Qw, sw, X.dtype, bias=bias)
    torch.cuda.synchronize()
    Qxr, sxr = orc.quantize_tensor(wl.X, dt)
    Qwr, swr = orc.quantize_tensor(wl.W, dt)
    C = orc.int8_rows(Qxr, Qwr, None)
    Yr = orc.output_rows(C, sxr, swr, wl.X, dt, np.zeros(0, np.int32), Qwr, wl.bias, None)
    check_y(bits_of(Y), Yr, dt, "per-tensor product")
