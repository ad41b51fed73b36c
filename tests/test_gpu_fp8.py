"""GPU parity of the FP8 (E4M3) variant against the CPU oracle.

Codes, scales, the outlier index list and count and XO must match bit for bit
(the quantization decisions are taken in the same fp32 arithmetic on both
sides).  The product C is accumulated by the matrix cores while the oracle's
is exact.  gfx950's fp8 dot-product instructions do not round each addition to
fp32.  Measured on this chip with crafted codes (one large product beside small
ones, through llmint8_matmul_fp8, both kernel families): the products of each
aligned group of 8 columns are added on a fixed-point grid of 2^(E-13), where
E is the group's largest exponent sum e(a) + e(b), smaller contributions
truncated (next to 448 x 448, E = 16, the grid is 8; next to 128 x 128,
E = 14, it is 2), and the group sums are then added into the fp32
accumulator.  The test's bound follows from that model:
  |C - C_exact| <= sum_groups 8 * 2^(E_g - 13) + (K/8 + 8) * 2^-24 * sum_k |a_k b_k|
(at most 8 truncations per group, then at most K/8 fp32 additions per lane and
8 more across waves).  Y must satisfy the same gate as the int8 path:
max|dY| <= 1e-2 * max|Y_ref| and, per element, ulp16(|Y_ref|) + 1e-4 max|Y_ref|.
"""
import numpy as np
import pytest

import pins
import synth
from gpu_helpers import bits_of, check_y, log, sample_rows, to_torch

pytestmark = pytest.mark.gpu

F16, BF16 = synth.F16, synth.BF16


@pytest.fixture(scope="module", autouse=True)
def gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import int8_quantized_matmul_row_amd as pkg
    pkg.lib()  # fails loudly when the library is missing


def run_gpu_fp8(wl, t, one_call=False, weight=None, device="cuda:0"):
    import torch
    import int8_quantized_matmul_row_amd as pkg
    dev = torch.device(device)
    X = to_torch(wl.X, wl.dtype, dev)
    if weight is None:
        CB, SCB = pkg.quantize_weight_fp8(to_torch(wl.W, wl.dtype, dev))
    else:
        CB, SCB = weight
    bias = None if wl.bias is None else to_torch(wl.bias, wl.dtype, dev)
    C = torch.empty((wl.M, wl.N), dtype=torch.float32, device=dev)
    if one_call:
        Y, q = pkg.linear_fp8(X, CB, SCB, bias=bias, threshold=t, C_f32=C)
    else:
        q = pkg.quantize_act_fp8(X, t)
        Y = pkg.matmul_fp8(q, CB, SCB, bias=bias, C_f32=C)
    torch.cuda.synchronize()
    n_out = int(q.n_out.item())
    n_pad = (n_out + 31) // 32 * 32
    return dict(CA=q.CA.cpu().numpy(), SCA=q.SCA.cpu().numpy(),
                idx=q.idx[:n_out].cpu().numpy(), n_out=n_out,
                XO=bits_of(q.XO[:wl.M * n_pad]).reshape(wl.M, n_pad),
                Y=bits_of(Y), C=C, weight=(CB, SCB))


def _exponent(codes):
    """Unbiased exponent of each E4M3 code (subnormals: -6); zeros very low."""
    e = np.maximum(((codes >> 3) & 15).astype(np.int32), 1) - 7
    return np.where((codes & 0x7F) == 0, -100000, e)


def c_bound(CA, CB, S, K):
    """The accumulation bound above, for rows CA [R,K] against CB [N,K]."""
    ea, eb = _exponent(CA), _exponent(CB)
    total = np.zeros((CA.shape[0], CB.shape[0]))
    for k0 in range(0, K, 8):
        E = (ea[:, None, k0:k0 + 8] + eb[None, :, k0:k0 + 8]).max(axis=-1)
        total += np.where(E > -50000, 8.0 * np.exp2(E - 13.0), 0.0)
    return total + (K / 8 + 8) * 2.0 ** -24 * S


def compare_fp8(orc, wl, g, ref, rows=None, label=""):
    n_out = g["n_out"]
    assert n_out == len(ref["idx"]), f"{label}: n_out {n_out} vs {len(ref['idx'])}"
    assert np.array_equal(g["idx"], ref["idx"]), f"{label}: outlier index list"
    assert np.array_equal(g["SCA"], ref["SCA"]), f"{label}: SCA"
    assert np.array_equal(g["CA"], ref["CA"]), f"{label}: CA codes"
    assert np.array_equal(g["XO"][:, :n_out], ref["XO"]), f"{label}: XO"
    assert not g["XO"][:, n_out:].any(), f"{label}: XO padding"
    sel = np.arange(wl.M) if rows is None else rows
    C = g["C"].cpu().numpy()[sel].astype(np.float64)
    S = orc.fp8_rows(ref["CA"] & 0x7F, ref["CB"] & 0x7F, sel)  # sum |a||b|
    err = np.abs(C - ref["C"])
    bound = c_bound(ref["CA"][sel], ref["CB"], S, wl.K)
    assert (err <= bound).all(), \
        f"{label}: C beyond the accumulation bound, worst {(err / np.maximum(bound, 1e-30)).max():.3g} x bound"
    return check_y(g["Y"][sel], ref["Y"], wl.dtype, label)


def full_check(orc, wl, t=None, rows=None, one_call=False, label=None):
    t = wl.threshold if t is None else t
    label = label or f"fp8 {wl.name} t={t}"
    log(f"[fp8] {label} M={wl.M} N={wl.N} K={wl.K} dtype={synth.DTYPE_NAMES[wl.dtype]}")
    g = run_gpu_fp8(wl, t, one_call=one_call)
    ref = orc.forward_fp8(wl.X, wl.W, wl.dtype, t, bias=wl.bias, rows=rows)
    CB, SCB = g["weight"]
    assert np.array_equal(CB.cpu().numpy(), ref["CB"]), f"{label}: CB codes"
    assert np.array_equal(SCB.cpu().numpy(), ref["SCB"]), f"{label}: SCB"
    err, scale = compare_fp8(orc, wl, g, ref, rows=rows, label=label)
    log(f"[fp8] {label}: ok, n_out={g['n_out']} max|dY|={err:.3g} max|Y|={scale:.3g}")
    return g, ref


# ---- weight codes: zero rows, negative zeros, both dtypes ---------------------
@pytest.mark.parametrize("N,K,dt", [(300, 1024, F16), (77, 4160, BF16)])
def test_fp8_weight_codes(orc, N, K, dt):
    import torch
    import int8_quantized_matmul_row_amd as pkg
    W = synth.normal_bits(5, 2, N, K, 0.05, dt)
    W[3] = 0
    W[4, ::3] = 0x8000               # -0.0 in both formats
    W[5] = 0x8000
    W[6, 7] = synth.to_bits(np.float32([300.0]), dt)[0]
    log(f"[fp8] weight codes N={N} K={K} dtype={synth.DTYPE_NAMES[dt]}")
    CB, SCB = pkg.quantize_weight_fp8(to_torch(W, dt, torch.device("cuda:0")))
    torch.cuda.synchronize()
    rCB, rSCB = orc.quantize_weight_fp8(W, dt)
    assert np.array_equal(SCB.cpu().numpy(), rSCB)
    assert np.array_equal(CB.cpu().numpy(), rCB)
    assert (rCB[5] == 0x80).all() and rCB[6, 7] == 0x7E


# ---- the decomposition over both kernel families, ragged shapes ---------------
RAGGED = [
    # M, N, K, dtype, planted outlier columns, bias
    (1, 1, 64, F16, 0, False),
    (3, 17, 128, BF16, 1, True),
    (8, 200, 4160, F16, 4, True),
    (16, 33, 192, F16, 2, True),
    (65, 40, 64, F16, 1, False),       # tiled, one stage
    (80, 64, 128, BF16, 2, True),      # tiled, two stages
    (40, 64, 128, BF16, 2, True),      # the streaming kernel, four groups of 16 rows
    (40, 16400, 128, F16, 36, True),   # ... in workgroups of 64 channels, many outlier columns
    (24, 16448, 192, BF16, 3, False),  # ... two groups of 16 rows, 64 channels
    (16, 16400, 128, F16, 2, True),    # ... one group of 16 rows, 64 channels
    (65, 300, 192, F16, 2, True),      # tiled, three stages
    (300, 520, 320, F16, 3, True),
    (300, 520, 320, BF16, 3, True),
    (257, 769, 448, BF16, 40, True),   # more than 16 outlier columns
    (513, 257, 1024, F16, 5, False),
    (37, 100, 8192, BF16, 3, True),    # 2 waves per activation row, odd M
]


@pytest.mark.parametrize("M,N,K,dt,nout,bias", RAGGED,
                         ids=[f"{r[0]}x{r[1]}x{r[2]}-{synth.DTYPE_NAMES[r[3]]}" for r in RAGGED])
def test_fp8_ragged_shapes(orc, M, N, K, dt, nout, bias):
    wl = synth.make_random(M, N, K, dt, seed=M + N + K + 1, n_outlier_cols=nout,
                           bias_sigma=0.01 if bias else None)
    full_check(orc, wl)


# ---- the fused decode kernel (the one-call forward at M <= 8, M*K <= 32768) ----
DECODE = [
    # M, N, K, dtype, planted outlier columns, bias, threshold
    (1, 1, 64, F16, 0, False, 6.0),
    (3, 17, 128, BF16, 1, True, 6.0),
    (8, 200, 4096, F16, 4, True, 6.0),     # all eight rows (the branch-free variant)
    (7, 64, 256, F16, 2, True, 6.0),
    (4, 300, 8192, BF16, 3, True, 6.0),    # two chunks per thread
    (8, 96, 512, F16, 2, False, 0.0),      # every column an outlier
    (8, 96, 512, BF16, 2, True, float("inf")),
]


@pytest.mark.parametrize("M,N,K,dt,nout,bias,t", DECODE,
                         ids=[f"{r[0]}x{r[1]}x{r[2]}-{synth.DTYPE_NAMES[r[3]]}-t{r[6]}" for r in DECODE])
def test_fp8_fused_decode(orc, M, N, K, dt, nout, bias, t):
    wl = synth.make_random(M, N, K, dt, seed=M * 7 + K, n_outlier_cols=nout,
                           bias_sigma=0.01 if bias else None)
    full_check(orc, wl, t=t, one_call=True, label=f"fp8 fused decode {M}x{N}x{K} t={t}")


@pytest.mark.parametrize("t", [0.0, float("inf"), 2.0])
@pytest.mark.parametrize("M", [8, 300])
def test_fp8_thresholds(orc, M, t):
    wl = synth.make_random(M, 96, 256, F16, seed=31, n_outlier_cols=3, bias_sigma=0.01)
    g, ref = full_check(orc, wl, t=t)
    if t == 0.0:
        assert g["n_out"] == 256 and not g["CA"].any() and not g["SCA"].any()
    if t == float("inf"):
        assert g["n_out"] == 0


# ---- one call against the two stages -------------------------------------------
# The activation results are the same bits either way.  At M <= 8 the one-call
# forward is the fused decode kernel, whose waves split K differently from the
# two-call GEMM, so the fp32 sums may round differently: both are held to the
# oracle.  At M > 16 both run the same kernels and agree bit for bit.
@pytest.mark.parametrize("M,N,K", [(8, 4096, 1024), (5, 300, 4096), (300, 520, 320)])
def test_fp8_linear_against_stages(orc, M, N, K):
    import torch
    wl = synth.make_random(M, N, K, F16, seed=41, n_outlier_cols=3, bias_sigma=0.01)
    a = run_gpu_fp8(wl, 6.0)
    b = run_gpu_fp8(wl, 6.0, one_call=True, weight=a["weight"])
    for key in ("CA", "SCA", "idx", "XO"):
        assert np.array_equal(a[key], b[key]), key
    ref = orc.forward_fp8(wl.X, wl.W, wl.dtype, 6.0, bias=wl.bias)
    compare_fp8(orc, wl, a, ref, label="two calls")
    compare_fp8(orc, wl, b, ref, label="one call")
    if M > 16:
        assert np.array_equal(a["Y"], b["Y"]) and torch.equal(a["C"], b["C"])


# ---- exact on E4M3-representable inputs (closed form) -------------------------
@pytest.mark.parametrize("seed,dt", [(0, F16), (1, BF16)])
def test_fp8_exact_inputs(seed, dt):
    import torch
    import int8_quantized_matmul_row_amd as pkg
    import bruteforce
    X, W, b, cols = pins.fp8_exact_case(seed, dt, M=20, N=300, K=512, n_out=5)
    dev = torch.device("cuda:0")
    CB, SCB = pkg.quantize_weight_fp8(to_torch(W, dt, dev))
    Y, q = pkg.linear_fp8(to_torch(X, dt, dev), CB, SCB, bias=to_torch(b, dt, dev), threshold=6.0)
    torch.cuda.synchronize()
    assert np.array_equal(q.idx[:int(q.n_out.item())].cpu().numpy(), cols)
    x = bruteforce.widen(X, dt).astype(np.float64)
    w = bruteforce.widen(W, dt).astype(np.float64)
    ref = x @ w.T + bruteforce.widen(b, dt).astype(np.float64)
    check_y(bits_of(Y), ref, dt, f"fp8 exact seed={seed}")


# ---- the fused decode kernel on the same exact inputs, with signed zeros --------
# Row 5's non-outlier entries are all +-0 (SCA = 0, scale 0); elsewhere -0 and
# +0 occur among the drawn values.  The codes keep the sign of a zero product
# (0x80 for -0), and Y is the closed form.
@pytest.mark.parametrize("seed,dt", [(0, F16), (1, BF16)])
def test_fp8_decode_exact_signed_zeros(orc, seed, dt):
    import torch
    import int8_quantized_matmul_row_amd as pkg
    import bruteforce
    X, W, b, cols = pins.fp8_exact_case(seed, dt, M=8, N=64, K=512, n_out=3)
    rest = np.setdiff1d(np.arange(512), cols)
    X[5, rest] = np.where(np.arange(rest.size) % 3 == 0, 0x8000, 0).astype(X.dtype)
    assert (X[:, rest] == 0x8000).sum() > 150
    dev = torch.device("cuda:0")
    CB, SCB = pkg.quantize_weight_fp8(to_torch(W, dt, dev))
    Y, q = pkg.linear_fp8(to_torch(X, dt, dev), CB, SCB, bias=to_torch(b, dt, dev), threshold=6.0)
    torch.cuda.synchronize()
    ref = orc.forward_fp8(X, W, dt, 6.0, bias=b)
    assert np.array_equal(q.idx[:int(q.n_out.item())].cpu().numpy(), cols)
    assert np.array_equal(q.SCA.cpu().numpy(), ref["SCA"]) and ref["SCA"][5] == 0.0
    ca = q.CA.cpu().numpy()
    assert np.array_equal(ca, ref["CA"])
    assert (ca.view(np.uint8)[5, rest] == 0x80).sum() == (X[5, rest] == 0x8000).sum()
    x = bruteforce.widen(X, dt).astype(np.float64)
    w = bruteforce.widen(W, dt).astype(np.float64)
    check_y(bits_of(Y), x @ w.T + bruteforce.widen(b, dt).astype(np.float64), dt,
            f"fp8 decode exact seed={seed}")


# ---- the full decode and prefill shapes, in the one-call launch ----------------
@pytest.mark.parametrize("name,nrows", [("decode", None), ("prefill", 6)])
def test_fp8_full_size(orc, name, nrows):
    wl = synth.make_workload(name)
    rows = None if nrows is None else sample_rows(wl.M, nrows, seed=3)
    full_check(orc, wl, rows=rows, one_call=True, label=f"fp8 {name} full size")
