"""Pins of the CPU oracle to facts fixed outside the oracle itself.

Each pin takes an oracle object and raises AssertionError on a mismatch.  The
pins are run against the real oracle (test_oracle_pins.py) and against copies
with planted mistakes (test_oracle_mutants.py), which must each fail at least
one pin.

Page titles cited:
  [GENTLE]  "A Gentle Introduction to 8-bit Matrix Multiplication for
            transformers at scale" (Chinese translation)
  [HF-INT8] "Hugging Face 将 LLM.int8() 8 位矩阵乘法集成到 Transformers 和
            Accelerate 中"
"""
from __future__ import annotations

import json
import os

import numpy as np

import synth
import bruteforce

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
F16, BF16 = synth.F16, synth.BF16


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _f16(vals):
    return synth.f32_to_f16_bits(np.asarray(vals, dtype=np.float32))


def _bf16(vals):
    return synth.f32_to_bf16_bits(np.asarray(vals, dtype=np.float32))


# -- P1: the worked absmax example ([GENTLE] "absmax quantization") ----------
def pin_absmax_worked_example(orc):
    g = _golden("absmax_worked_example.json")
    exp = np.array(g["expected_int8"], dtype=np.int8)
    # fp16 holds the printed values closely enough to keep every code; bf16
    # (8 mantissa bits) turns 2.4 into 2.40625 and 5.4 into 5.40625, which moves
    # the seventh code to 57, so the example is checked on fp16 inputs only.
    for dt, conv in ((F16, _f16),):
        bits = conv(g["input"]).reshape(1, -1)
        CB, SCB = orc.quantize_weight(bits, dt)
        assert np.array_equal(CB[0], exp), (dt, CB[0], exp)
        assert abs(float(SCB[0]) - g["absmax"]) < 0.02
        assert abs(127.0 / float(SCB[0]) - g["scale_approx"]) < 0.1
        # the same vector as one activation row with no outliers
        CA, SCA, idx, _ = orc.quantize_act(bits, dt, float("inf"))
        assert np.array_equal(CA[0], exp) and idx.size == 0
        assert SCA[0] == SCB[0]


# -- P2: the fixed-range example ([GENTLE] "zero-point quantization") --------
def pin_zero_point_example(orc):
    g = _golden("zero_point_example.json")
    W = _f16([[g["value"], g["range_absmax"]]])
    CB, SCB = orc.quantize_weight(W, F16)
    assert int(CB[0, 0]) == g["quantized"] and int(CB[0, 1]) == 127
    rec = orc.recover_weight(CB, SCB)
    assert round(float(rec[0, 0]), 4) == g["recovered_4dp"]
    # the recovered value reaches the output through the outlier product:
    # a one-hot activation at threshold 0 returns the recovered weight row.
    X = _f16([[1.0, 0.0]])
    out = orc.forward(X, W, F16, 0.0, weight=(CB, SCB))
    assert round(float(out["Y"][0, 0]), 4) == g["recovered_4dp"]


# -- P3: the printed 64x64 layer ([GENTLE] "Usage") -------------------------
def pin_usage_printouts(orc):
    g = _golden("usage_weight_printouts.json")
    W = np.array(g["weight_fp16"], dtype=np.float64)
    CBp = np.array(g["weight_int8"], dtype=np.int64)
    R = np.array(g["recovered_print"], dtype=np.float64)
    # the third print is CB * SCB broadcast over the last axis: column j gives SCB[j]
    ratios = R * 127.0 / CBp
    scb = np.median(ratios, axis=0)
    assert np.all(np.abs(ratios - scb) <= 0.0051), "recovered print is not CB*SCB[col]/127"
    # visible row r's absmax is SCB[r]; rebuild each visible row with that maximum
    n_in = g["in_features"]
    rows = np.zeros((len(g["rows"]), n_in), dtype=np.float32)
    rows[:, g["cols"]] = W
    rows[:, 30] = scb  # an unseen entry holding the row maximum
    CB, _ = orc.quantize_weight(_f16(rows), F16)
    got = CB[:, g["cols"]].astype(np.int64)
    assert np.abs(got - CBp).max() <= 1, (got, CBp)
    assert (got == CBp).sum() >= 34, (got == CBp).sum()


# -- P4: round half to even on a designed row (exact ties) ------------------
def pin_round_half_even(orc):
    # absmax 3.96875 = 127/32, so the scale is exactly 32 and x*32 lands on ties
    row = [3.96875, 0.078125, 0.015625, 0.046875, -0.078125, 0.109375]
    exp = np.array([127, 2, 0, 2, -2, 4], dtype=np.int8)
    CB, SCB = orc.quantize_weight(_f16([row]), F16)
    assert np.array_equal(CB[0], exp), CB[0]
    CA, SCA, _, _ = orc.quantize_act(_f16([row]), F16, 6.0)
    assert np.array_equal(CA[0], exp), CA[0]


# -- P5: the threshold boundary ([GENTLE] "inside the MatMul": 6 or greater) -
def pin_threshold_boundary(orc):
    X = np.zeros((3, 8), dtype=np.float32)
    X[1, 2] = 6.0            # exactly the threshold: outlier
    X[2, 5] = -6.0           # negative, magnitude 6: outlier
    X[0, 6] = 5.99609375     # the fp16 just below 6: not an outlier
    X[0, 0] = 1.0
    CA, SCA, idx, XO = orc.quantize_act(_f16(X), F16, 6.0)
    assert list(idx) == [2, 5], idx
    assert CA[1, 2] == 0 and CA[2, 5] == 0
    assert SCA[0] == np.float32(5.99609375) and CA[0, 6] == 127
    assert SCA[1] == 0 and SCA[2] == 0        # rows whose only mass is outlier
    assert np.array_equal(synth.bits_to_f32(XO, F16)[:, 0], [0, 6.0, 0])


# -- P6: threshold +inf reduces to plain vector-wise int8 --------------------
def pin_threshold_inf_closed_form(orc):
    wl = synth.make_random(12, 10, 64, F16, seed=3, n_outlier_cols=2, bias_sigma=0.01)
    out = orc.forward(wl.X, wl.W, F16, float("inf"), bias=wl.bias)
    assert out["idx"].size == 0
    x = bruteforce.widen(wl.X, F16)
    CA, SCA = bruteforce.absmax_quantize_rows(x)
    assert np.array_equal(out["CA"], CA) and np.array_equal(out["SCA"], SCA)
    C = out["CA"].astype(np.int64) @ out["CB"].astype(np.int64).T
    Y = C * np.outer(out["SCA"].astype(np.float64), out["SCB"].astype(np.float64)) / 127.0**2
    Y += bruteforce.widen(wl.bias, F16).astype(np.float64)
    assert np.allclose(out["Y"], Y, rtol=1e-12, atol=1e-12)
    # on data with no |x| >= 6 the thresholds 6 and +inf agree at every stage
    clean = synth.make_random(12, 10, 64, F16, seed=4)
    a = orc.forward(clean.X, clean.W, F16, 6.0)
    b = orc.forward(clean.X, clean.W, F16, float("inf"))
    for key in ("CA", "SCA", "idx", "C", "Y"):
        assert np.array_equal(a[key], b[key]), key


# -- P7: threshold 0 makes every column an outlier: Y = X . Wdq^T + bias -----
def pin_threshold_zero_closed_form(orc):
    wl = synth.make_random(9, 11, 64, F16, seed=5, n_outlier_cols=3, bias_sigma=0.01)
    out = orc.forward(wl.X, wl.W, F16, 0.0, bias=wl.bias)
    assert np.array_equal(out["idx"], np.arange(64))
    assert not out["CA"].any() and not out["SCA"].any() and not out["C"].any()
    Wdq = out["CB"].astype(np.float64) * out["SCB"].astype(np.float64)[:, None] / 127.0
    Y = bruteforce.widen(wl.X, F16).astype(np.float64) @ Wdq.T
    Y += bruteforce.widen(wl.bias, F16).astype(np.float64)
    assert np.allclose(out["Y"], Y, rtol=1e-12, atol=1e-13)


# -- P8: brute force on tiny inputs, every stage -----------------------------
def compare_with_bruteforce(orc, X, W, dtype, t, bias=None):
    ref = bruteforce.forward(X, W, dtype, t, bias)
    out = orc.forward(X, W, dtype, t, bias=bias)
    for key in ("CB", "SCB", "CA", "SCA", "idx", "XO", "C"):
        assert np.array_equal(out[key], ref[key]), key
    assert np.allclose(out["Y"], ref["Y"], rtol=1e-12, atol=1e-12)


def pin_bruteforce_tiny(orc):
    rng = np.random.default_rng([7, 0])
    for trial in range(40):
        M, N, K = (int(v) for v in rng.integers(1, 9, size=3))
        dt = F16 if trial % 2 == 0 else BF16
        conv = _f16 if dt == F16 else _bf16
        X = conv(rng.normal(0, 3.0, (M, K)).astype(np.float32))
        W = conv(rng.normal(0, 0.05, (N, K)).astype(np.float32))
        bias = conv(rng.normal(0, 0.1, N).astype(np.float32)) if trial % 3 == 0 else None
        t = [6.0, 2.0, 0.0, float("inf")][trial % 4]
        compare_with_bruteforce(orc, X, W, dt, t, bias)


# -- P9: invariants ----------------------------------------------------------
def pin_invariants(orc):
    wl = synth.make_random(6, 5, 64, F16, seed=9, n_outlier_cols=2)
    base = orc.forward(wl.X, wl.W, F16, 6.0)
    # jointly permuting K permutes CA, CB and the outlier set; SCA, SCB, C fixed
    perm = np.random.default_rng([9, 1]).permutation(64)
    p = orc.forward(wl.X[:, perm], wl.W[:, perm], F16, 6.0)
    assert np.array_equal(p["CA"], base["CA"][:, perm])
    assert np.array_equal(p["CB"], base["CB"][:, perm])
    assert np.array_equal(p["SCA"], base["SCA"]) and np.array_equal(p["SCB"], base["SCB"])
    assert np.array_equal(p["C"], base["C"])
    assert np.array_equal(np.sort(perm[p["idx"]]), base["idx"])
    # scaling a weight row by 2^j leaves CB alone and scales SCB by 2^j
    w = bruteforce.widen(wl.W, F16).copy()
    w[2] *= np.float32(4.0)
    CB2, SCB2 = orc.quantize_weight(_f16(w), F16)
    assert np.array_equal(CB2, base["CB"]) and SCB2[2] == 4 * base["SCB"][2]
    # with no outliers, scaling an activation row by 2^j scales only its SCA
    x = bruteforce.widen(wl.X, F16).copy()
    CA0, SCA0, _, _ = orc.quantize_act(_f16(x), F16, float("inf"))
    x[3] *= np.float32(0.5)
    CA1, SCA1, _, _ = orc.quantize_act(_f16(x), F16, float("inf"))
    assert np.array_equal(CA0, CA1) and SCA1[3] == SCA0[3] / 2
    # the int32 bound |C| <= K * 127^2
    assert np.abs(base["C"].astype(np.int64)).max() <= 64 * 127 * 127


# -- P10: per-tensor absmax, the baseline scheme ([GENTLE] "absmax
# quantization": one scale 127/absmax for the whole vector or tensor) -------
def _tensor_bruteforce(bits, dt):
    """numpy float32 arithmetic: amax over the tensor, s = 127/amax in float32,
    q = rint(x * s) (round half to even), clamped."""
    a = bruteforce.widen(bits, dt).astype(np.float32)
    amax = np.float32(np.abs(a).max()) if a.size else np.float32(0)
    if amax == 0:
        return np.zeros(a.shape, np.int8), np.full(a.shape[0], amax, np.float32)
    s = np.float32(127.0) / amax
    q = np.clip(np.rint((a * s).astype(np.float32)), -127, 127).astype(np.int8)
    return q, np.full(a.shape[0], amax, np.float32)


def pin_per_tensor_absmax(orc):
    # the worked example, read as a one-row tensor
    g = _golden("absmax_worked_example.json")
    Q, scale = orc.quantize_tensor(_f16(g["input"]).reshape(1, -1), F16)
    assert np.array_equal(Q[0], np.array(g["expected_int8"], dtype=np.int8))
    # brute force on tensors whose rows have different maxima
    rng = np.random.default_rng([10, 0])
    for trial in range(20):
        R, C = (int(v) for v in rng.integers(1, 9, size=2))
        dt = F16 if trial % 2 == 0 else BF16
        conv = _f16 if dt == F16 else _bf16
        A = conv(rng.normal(0, 1.0, (R, C)).astype(np.float32) *
                 rng.uniform(0.1, 10.0, (R, 1)).astype(np.float32))
        Q, scale = orc.quantize_tensor(A, dt)
        Qb, sb = _tensor_bruteforce(A, dt)
        assert np.array_equal(Q, Qb) and np.array_equal(scale, sb), (trial, R, C)
    # rows that all share one absmax: per-tensor equals per-row (vector-wise)
    x = np.array([[1.0, -3.0, 0.5], [3.0, 2.0, -1.25]], dtype=np.float32)
    Q, scale = orc.quantize_tensor(_f16(x), F16)
    CB, SCB = orc.quantize_weight(_f16(x), F16)
    assert np.array_equal(Q, CB) and np.array_equal(scale, SCB)
    # an all-zero tensor
    Q, scale = orc.quantize_tensor(np.zeros((3, 4), np.uint16), F16)
    assert not Q.any() and not scale.any()


ALL_PINS = [
    pin_absmax_worked_example,
    pin_zero_point_example,
    pin_usage_printouts,
    pin_round_half_even,
    pin_threshold_boundary,
    pin_threshold_inf_closed_form,
    pin_threshold_zero_closed_form,
    pin_bruteforce_tiny,
    pin_invariants,
    pin_per_tensor_absmax,
]
