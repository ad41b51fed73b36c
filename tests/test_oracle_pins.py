"""The CPU oracle against what the pages and the mathematics fix (no GPU)."""
import numpy as np
import pytest

import pins
import synth


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)


@pytest.mark.parametrize("M,N,K", [(m, n, k) for m in range(1, 9) for n in range(1, 9)
                                   for k in range(1, 9)])
def test_bruteforce_all_tiny_shapes(orc, M, N, K):
    """Every M, N, K in 1..8 against the independent numpy brute force."""
    rng = np.random.default_rng([11, M, N, K])
    X = synth.f32_to_f16_bits(rng.normal(0, 3.0, (M, K)).astype(np.float32))
    W = synth.f32_to_f16_bits(rng.normal(0, 0.05, (N, K)).astype(np.float32))
    bias = synth.f32_to_f16_bits(rng.normal(0, 0.1, N).astype(np.float32))
    pins.compare_with_bruteforce(orc, X, W, synth.F16, 6.0, bias)


def test_tiny_workload_outlier_set(orc):
    """The tiny workload's planted columns 7 and 500 are the detected outliers."""
    wl = synth.make_workload("tiny")
    CA, SCA, idx, XO = orc.quantize_act(wl.X, wl.dtype, wl.threshold)
    assert list(idx) == [7, 500]
    assert np.all(np.abs(synth.bits_to_f32(XO, wl.dtype)) == 20.0)


def test_decomposition_reduces_error(orc):
    """The method's purpose: with outliers present, threshold 6 is far closer to
    the exact product than plain vector-wise int8 (threshold +inf).  A property
    of the method, not a pinned figure: the pages print no matmul-level error."""
    wl = synth.make_workload("tiny")
    x = synth.bits_to_f32(wl.X, wl.dtype).astype(np.float64)
    w = synth.bits_to_f32(wl.W, wl.dtype).astype(np.float64)
    exact = x @ w.T
    e6 = np.abs(orc.forward(wl.X, wl.W, wl.dtype, 6.0)["Y"] - exact).max()
    einf = np.abs(orc.forward(wl.X, wl.W, wl.dtype, float("inf"))["Y"] - exact).max()
    assert e6 * 3 < einf, (e6, einf)


def test_bf16_and_fp16_widening_exact(orc):
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    f16 = orc.widen(bits, synth.F16)
    ref = bits.view(np.float16).astype(np.float32)
    same = (f16 == ref) | (np.isnan(f16) & np.isnan(ref))
    assert same.all()
    bf = orc.widen(bits, synth.BF16)
    ref = (bits.astype(np.uint32) << 16).view(np.float32)
    assert ((bf == ref) | (np.isnan(bf) & np.isnan(ref))).all()


def test_rejects_bad_arguments(orc):
    import oracle
    X = synth.f32_to_f16_bits(np.ones((2, 4), np.float32))
    with pytest.raises(oracle.OracleError):
        orc.quantize_act(X, synth.F16, float("nan"))
    with pytest.raises(oracle.OracleError):
        orc.quantize_act(X, synth.F16, -1.0)
    bad = X.copy()
    bad[0, 0] = 0x7C00  # +inf
    with pytest.raises(oracle.OracleError):
        orc.quantize_act(bad, synth.F16, 6.0)
