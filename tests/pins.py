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
  [ZHICHAI] the zhichai.top summary of LLM.int8(), outlook section ("未来展望"),
            which names an 8-bit floating-point type as future work; the FP8
            pins (P11-P15) fix the E4M3 reading of it against torch's
            float8_e4m3fn casts, integer arithmetic and exact closed forms.
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


# -- FP8 (E4M3) variant ([ZHICHAI] "未来展望") ---------------------------------
def _torch_e4m3(x):
    """float32 -> E4M3 codes by torch's float8_e4m3fn cast (a library routine:
    nearest, ties to even, NaN beyond the finite range)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _torch_e4m3_values(codes):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8))
    return t.view(torch.float8_e4m3fn).to(torch.float32).numpy().astype(np.float64)


# -- P11: the code book and the rounding of E4M3 ------------------------------
def pin_e4m3_codec(orc):
    codes = np.arange(256, dtype=np.uint8)
    ref = _torch_e4m3_values(codes)
    got = orc.e4m3_decode(codes)
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all(), np.nonzero(~same)
    assert np.isnan(got[[0x7F, 0xFF]]).all() and np.isnan(got).sum() == 2
    assert got[0x7E] == 448.0 and got[0x08] == 2.0 ** -6 and got[0x01] == 2.0 ** -9
    assert got[0x38] == 1.0 and np.signbit(got[0x80])
    # encoding: every finite code, every midpoint between neighbours (ties),
    # a float32 ulp either side of each midpoint, log-uniform random values
    # from far below the smallest subnormal to beyond the largest finite value
    fin = np.sort(np.unique(got[np.isfinite(got) & (got >= 0)]))
    mid = ((fin[1:] + fin[:-1]) / 2).astype(np.float32)
    rng = np.random.default_rng([11, 0])
    rnd = (2.0 ** rng.uniform(-13, 8.9, 20000)).astype(np.float32)
    pos = np.concatenate([fin.astype(np.float32), mid, np.nextafter(mid, np.float32(0)),
                          np.nextafter(mid, np.float32(np.inf)), rnd, np.float32([456.0, 463.9])])
    x = np.concatenate([pos, -pos, np.float32([0.0, -0.0])])
    e = orc.e4m3_encode(x)
    r = _torch_e4m3(x)
    assert np.array_equal(e, r), x[e != r][:10]
    # and by search: the encoded value is a nearest finite value; at a tie the
    # code with the even mantissa field wins
    v = got[e[:4000].astype(np.int64)]
    for xi, vi, ci in zip(x[:4000].astype(np.float64), v, e[:4000]):
        if not np.isfinite(vi):
            continue
        d = np.abs(got[np.isfinite(got)] - xi).min()
        assert abs(vi - xi) == d, (xi, vi)
    assert orc.e4m3_encode(np.float32([480.0]))[0] == 0x7F  # no finite code


# -- P12: weight quantization to E4M3 ----------------------------------------
def pin_fp8_weight(orc):
    rng = np.random.default_rng([12, 0])
    for trial, dt in enumerate((F16, BF16, F16)):
        conv = _f16 if dt == F16 else _bf16
        N, K = 7, 96
        w = rng.normal(0, 0.05, (N, K)).astype(np.float32) * rng.uniform(0.1, 20, (N, 1)).astype(np.float32)
        w[3] = 0.0
        w[4, ::2] = -0.0
        w[5, :] = 0.0
        w[5, 10] = -2.0 ** -20
        bits = conv(w)
        CB, SCB = orc.quantize_weight_fp8(bits, dt)
        a = bruteforce.widen(bits, dt).astype(np.float32)
        amax = np.abs(a).max(axis=1).astype(np.float32)
        assert np.array_equal(SCB, amax), trial
        for n in range(N):
            s = np.float32(448.0) / amax[n] if amax[n] > 0 else np.float32(0.0)
            exp = _torch_e4m3((a[n] * s).astype(np.float32))
            assert np.array_equal(CB[n], exp), (trial, n)
            if amax[n] > 0:  # the row maximum becomes +-448
                k = int(np.argmax(np.abs(a[n])))
                assert CB[n, k] in (0x7E, 0xFE), (trial, n, CB[n, k])
        assert not (CB[3] & 0x7F).any() and (CB[4, ::2] == 0x80).all()
        # the recovered weight is within half an E4M3 step of the weight
        vals = orc.e4m3_decode(CB) * SCB[:, None].astype(np.float64) / 448.0
        step = np.maximum(np.abs(a) * 2.0 ** -4, amax[:, None] / 448.0 * 2.0 ** -10)
        assert (np.abs(vals - a) <= step * (1 + 1e-9)).all()


# -- P13: activation quantization to E4M3 ------------------------------------
def pin_fp8_activation(orc):
    wl = synth.make_random(9, 4, 128, F16, seed=13, n_outlier_cols=3)
    for t in (6.0, 2.0, 0.0, float("inf")):
        CA, SCA, idx, XO = orc.quantize_act_fp8(wl.X, F16, t)
        # the outlier split and the row scales do not depend on the code format
        CAi, SCAi, idxi, XOi = orc.quantize_act(wl.X, F16, t)
        assert np.array_equal(idx, idxi) and np.array_equal(XO, XOi)
        assert np.array_equal(SCA, SCAi)
        a = bruteforce.widen(wl.X, F16).astype(np.float32)
        keep = np.ones(128, bool)
        keep[idx] = False
        for m in range(9):
            s = np.float32(448.0) / SCA[m] if SCA[m] > 0 else np.float32(0.0)
            exp = _torch_e4m3((a[m] * s).astype(np.float32))
            exp[~keep] = 0
            assert np.array_equal(CA[m], exp), (t, m)
            if SCA[m] > 0:
                k = int(np.argmax(np.where(keep, np.abs(a[m]), -1)))
                assert CA[m, k] in (0x7E, 0xFE)


# -- P14: the FP8 product, exact, by integer arithmetic ----------------------
def pin_fp8_product(orc):
    rng = np.random.default_rng([14, 0])
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    for M, N, K in ((3, 5, 64), (1, 1, 1), (4, 2, 8192)):
        CA = rng.choice(finite, (M, K)).astype(np.uint8)
        CB = rng.choice(finite, (N, K)).astype(np.uint8)
        if K == 8192:  # the largest sum: every product 448^2, one sign
            CA[0] = 0x7E
            CB[0] = 0x7E
        C = orc.fp8_rows(CA, CB)
        ia = np.rint(_torch_e4m3_values(CA) * 512).astype(np.int64)  # multiples of 2^-9
        ib = np.rint(_torch_e4m3_values(CB) * 512).astype(np.int64)
        exact = ia @ ib.T
        assert np.array_equal(C * 2.0 ** 18, exact.astype(np.float64)), (M, N, K)
    rows = np.array([2, 0], dtype=np.int64)
    assert np.array_equal(orc.fp8_rows(CA, CB, rows), orc.fp8_rows(CA, CB)[rows])


# -- P15: the FP8 output is exact on E4M3-representable inputs ---------------
def fp8_exact_case(seed, dt, M=6, N=5, K=128, n_out=3, bias=True):
    """X, W whose non-outlier rows are E4M3 values times a power of two with
    each row's maximum at 448 times that power, so that every code and every
    scale is exact and the method returns X . W^T + bias exactly."""
    rng = np.random.default_rng([15, seed])
    conv = _f16 if dt == F16 else _bf16
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = _torch_e4m3_values(finite)
    cols = rng.choice(K, n_out, replace=False)
    rest = np.setdiff1d(np.arange(K), cols)
    w = rng.choice(vals, (N, K)) * 2.0 ** -6
    w[np.arange(N), rng.integers(0, K, N)] = 448.0 * 2.0 ** -6 * rng.choice([-1, 1], N)
    x = rng.choice(vals, (M, K)) * 2.0 ** -7          # |x| <= 3.5 < 6
    x[np.arange(M), rng.choice(rest, M)] = 448.0 * 2.0 ** -7 * rng.choice([-1, 1], M)
    x[:, cols] = rng.uniform(-3, 3, (M, n_out))
    x[0, cols] = rng.choice([-1, 1], n_out) * rng.uniform(6, 40, n_out)
    X, W = conv(x.astype(np.float32)), conv(w.astype(np.float32))
    b = conv(rng.normal(0, 0.5, N).astype(np.float32)) if bias else None
    return X, W, b, np.sort(cols)


def pin_fp8_exact_closed_form(orc):
    for seed, dt in ((0, F16), (1, BF16), (2, F16)):
        X, W, b, cols = fp8_exact_case(seed, dt, bias=seed != 2)
        out = orc.forward_fp8(X, W, dt, 6.0, bias=b)
        assert np.array_equal(out["idx"], cols)
        x = bruteforce.widen(X, dt).astype(np.float64)
        w = bruteforce.widen(W, dt).astype(np.float64)
        ref = x @ w.T + (bruteforce.widen(b, dt).astype(np.float64) if b is not None else 0.0)
        assert np.allclose(out["Y"], ref, rtol=1e-12, atol=1e-12), np.abs(out["Y"] - ref).max()
        # threshold +inf: the outlier columns go through E4M3 too and are no
        # longer exact; the error is bounded by the codes' half step
        inf = orc.forward_fp8(X, W, dt, float("inf"), bias=b)
        assert inf["idx"].size == 0 and not np.allclose(inf["Y"], ref, rtol=1e-12, atol=1e-12)


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
    pin_e4m3_codec,
    pin_fp8_weight,
    pin_fp8_activation,
    pin_fp8_product,
    pin_fp8_exact_closed_form,
]
