"""GPU parity: the HIP path through the C-ABI against the CPU oracle.

Integer stages (CB, SCB, CA, SCA, the outlier index list and count, XO, the
int32 accumulators) must match bit for bit; Y must satisfy
max|dY| <= 1e-2 * max|Y_ref| and, per element, |dY| <= ulp16(|Y_ref|) +
1e-4 * max|Y_ref| (the 16-bit output rounding plus fp32 evaluation error).
"""
import numpy as np
import pytest

import synth
from gpu_helpers import compare, host_threads, log, oracle_forward, run_gpu, sample_rows

pytestmark = pytest.mark.gpu

F16, BF16 = synth.F16, synth.BF16


@pytest.fixture(scope="module", autouse=True)
def gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import int8_quantized_matmul_row_amd as pkg
    pkg.lib()  # fails loudly when the library is missing


@pytest.fixture(params=["256", "224"], ids=["w256", "w224"])
def tile_cols(request, monkeypatch):
    """The tiled product's tile width, forced (LLMINT8_TILE_COLS): both
    kernels' ragged edges, splits and outlier paths get the small shapes."""
    monkeypatch.setenv("LLMINT8_TILE_COLS", request.param)
    return int(request.param)


def full_check(orc, wl, threshold=None, label=None):
    t = wl.threshold if threshold is None else threshold
    label = label or f"{wl.name} t={t}"
    log(f"[parity] {label} M={wl.M} N={wl.N} K={wl.K} dtype={synth.DTYPE_NAMES[wl.dtype]}")
    g = run_gpu(wl, t)
    ref = orc.forward(wl.X, wl.W, wl.dtype, t, bias=wl.bias)
    err, scale = compare(wl, g, ref, label=label)
    log(f"[parity] {label}: ok, n_out={g['n_out']} max|dY|={err:.3g} max|Y|={scale:.3g}")
    return g, ref


# ---- the small named workloads, every row ----------------------------------
@pytest.mark.parametrize("name", ["tiny", "decode", "batch_32"])
def test_named_workload_full(orc, name):
    wl = synth.make_workload(name)
    g, ref = full_check(orc, wl)
    if name == "tiny":
        assert list(ref["idx"]) == [7, 500]


# ---- ragged shapes over both kernel families -------------------------------
RAGGED = [
    # M, N, K, dtype, planted outlier columns, bias
    (1, 1, 64, F16, 0, False),
    (3, 17, 128, BF16, 1, True),
    (8, 4100, 256, F16, 2, True),
    (16, 33, 192, F16, 2, True),
    (17, 40, 64, F16, 1, False),
    (65, 40, 64, F16, 1, False),
    # the streaming kernel's two and four groups of 16 token rows, with more
    # than 32 outlier columns (their product as 16-bit MFMAs) and without
    (30, 130, 512, F16, 36, False),
    (48, 200, 1024, BF16, 40, True),
    (64, 96, 2048, F16, 3, True),
    # workgroups of 64 channels (N >= 16384), two and four groups of 16 token
    # rows, a ragged last workgroup, with and without many outlier columns
    (40, 16400, 128, F16, 36, True),
    (20, 16448, 192, BF16, 3, False),
    (64, 16384, 256, F16, 0, True),
    (12, 16400, 256, F16, 36, True),    # one group of 16 rows, 64 channels
    (9, 16448, 128, BF16, 2, False),
    (5, 16448, 128, BF16, 2, False),    # up to 8 rows: 16 channels
    (300, 520, 320, F16, 3, True),
    (300, 520, 320, BF16, 3, True),
    (513, 257, 1024, F16, 5, False),
    (257, 769, 448, BF16, 40, True),
    (80, 64, 57344, BF16, 2, False),
    (8, 96, 133120, F16, 1, False),
    # few long rows: the activation kernel shares each row among 2 or 4 waves
    (37, 100, 8192, BF16, 3, True),     # 2 waves per row, odd M (a half-empty row group)
    (50, 70, 12352, F16, 5, False),     # 4 waves per row, one batch each
    (21, 40, 20480, F16, 2, True),      # 4 waves per row, the last with no batch
    # the tiled product's K split in 4, the last part ending in a half (64-byte) stage
    (300, 700, 4160, F16, 20, True),
]


@pytest.mark.parametrize("M,N,K,dt,nout,bias", RAGGED,
                         ids=[f"{r[0]}x{r[1]}x{r[2]}-{synth.DTYPE_NAMES[r[3]]}" for r in RAGGED])
def test_ragged_shapes(orc, M, N, K, dt, nout, bias, tile_cols):
    if M <= 64 and tile_cols == 224:
        pytest.skip("M <= 64: the small-M kernels, no tiles")
    wl = synth.make_random(M, N, K, dt, seed=M + N + K, n_outlier_cols=nout,
                           bias_sigma=0.01 if bias else None)
    full_check(orc, wl)


# ---- degenerate cases the method has ----------------------------------------
@pytest.mark.parametrize("M,N,K", [(8, 100, 256), (64, 300, 512),
                                   (16, 130, 4096)])  # the small-M product over 4096 outlier columns
def test_threshold_zero_every_column_outlier(orc, M, N, K, tile_cols):
    wl = synth.make_random(M, N, K, F16, seed=21, n_outlier_cols=2, bias_sigma=0.01)
    g, ref = full_check(orc, wl, threshold=0.0)
    assert g["n_out"] == K and not g["CA"].any() and not g["SCA"].any()
    assert not g["C_dev"].any().item()


@pytest.mark.parametrize("M,N,K", [(8, 100, 256), (64, 300, 512)])
def test_threshold_inf_no_outliers(orc, M, N, K, tile_cols):
    wl = synth.make_random(M, N, K, BF16, seed=22, n_outlier_cols=3)
    g, _ = full_check(orc, wl, threshold=float("inf"))
    assert g["n_out"] == 0


# ---- more than 16 outlier columns: codes gathered into the workspace --------
MANY = [
    # M, N, K, dtype, planted outlier columns, threshold (None: the default)
    (257, 769, 448, BF16, 40, None),
    (72, 33, 576, F16, 150, None),
    (300, 100, 1024, F16, 0, 0.0),   # every column: 1024 > the default capacity
]


@pytest.mark.parametrize("fp8", [False, True], ids=["int8", "fp8"])
@pytest.mark.parametrize("M,N,K,dt,nout,t", MANY,
                         ids=[f"{r[0]}x{r[1]}x{r[2]}-{r[4]}" for r in MANY])
def test_gathered_outlier_codes_match_direct_gathers(M, N, K, dt, nout, t, fp8, tile_cols):
    """The tiled product gives the same bits whether its outlier K loop reads
    the weight codes gathered into the workspace (default and full-capacity
    workspaces) or the plain kernel gathers them per tile (no workspace, one
    too small, or C exported)."""
    import torch
    import int8_quantized_matmul_row_amd as pkg
    from gpu_helpers import to_torch
    wl = synth.make_random(M, N, K, dt, seed=5 * M + N, n_outlier_cols=nout, bias_sigma=0.01)
    t = wl.threshold if t is None else t
    dev = torch.device("cuda:0")
    X, W = to_torch(wl.X, dt, dev), to_torch(wl.W, dt, dev)
    bias = to_torch(wl.bias, dt, dev)
    if fp8:
        CB, SCB = pkg.quantize_weight_fp8(W)
        q = pkg.quantize_act_fp8(X, t)
        mm = pkg.matmul_fp8
    else:
        CB, SCB = pkg.quantize_weight(W)
        q = pkg.quantize_act(X, t)
        mm = pkg.matmul
    n_out = int(q.n_out.item())
    log(f"[parity] gathered outlier codes {M}x{N}x{K} fp8={fp8} n_out={n_out} tile columns {tile_cols}")
    assert n_out > 16
    default_bytes = pkg.llmint8_matmul_workspace_size(M, N, K)
    full_bytes = N * K                # every column
    small_bytes = 64 * N - 1          # holds no 64-column group
    runs = {}
    for name, nbytes in [("none", 0), ("small", small_bytes), ("default", default_bytes),
                         ("full", full_bytes)]:
        ws = torch.full((max(nbytes, 1),), 0x5A, dtype=torch.uint8, device=dev)  # stale bytes
        Y = mm(q, CB, SCB, bias=bias, workspace=(ws if nbytes else None, nbytes))
        runs[name] = Y.view(torch.int16).cpu()
    # exporting C moves the call to the kernel that gathers the codes itself
    C = torch.empty((M, N), dtype=torch.float32 if fp8 else torch.int32, device=dev)
    ws = torch.empty((max(default_bytes, 1),), dtype=torch.uint8, device=dev)
    ckw = {"C_f32": C} if fp8 else {"C_i32": C}
    runs["export"] = mm(q, CB, SCB, bias=bias, workspace=(ws, default_bytes), **ckw).view(torch.int16).cpu()
    for name in ("small", "default", "full", "export"):
        assert torch.equal(runs[name], runs["none"]), name
    # the one-call forward: codes gathered by the activation kernel (default
    # workspace), or by the product's own gather kernel (a workspace holding
    # more columns than the activation kernel lists)
    lin = pkg.linear_fp8 if fp8 else pkg.linear
    lin_size = (pkg.llmint8_linear_fp8_workspace_size if fp8 else pkg.llmint8_linear_workspace_size)
    base = lin_size(M, N, K)
    for extra in (0, full_bytes - default_bytes):
        ws = torch.full((base + extra,), 0x5A, dtype=torch.uint8, device=dev)
        Y, _ = lin(X, CB, SCB, bias=bias, threshold=t, workspace=(ws, base + extra))
        assert torch.equal(Y.view(torch.int16).cpu(), runs["none"]), extra
    # and a second call with fewer outlier columns into the same (stale) workspace
    if t != 0.0:
        X2 = X.clone()
        X2[:, q.idx[:n_out // 2].long()] = 0   # half the outlier columns drop out
        q2 = (pkg.quantize_act_fp8 if fp8 else pkg.quantize_act)(X2, t)
        assert 16 < int(q2.n_out.item()) < n_out
        ws = torch.empty((default_bytes,), dtype=torch.uint8, device=dev)
        Y1 = mm(q, CB, SCB, bias=bias, workspace=(ws, default_bytes))
        Y2 = mm(q2, CB, SCB, bias=bias, workspace=(ws, default_bytes))
        Y2_none = mm(q2, CB, SCB, bias=bias, workspace=(None, 0))
        assert torch.equal(Y1.view(torch.int16).cpu(), runs["none"])
        assert torch.equal(Y2.view(torch.int16).cpu(), Y2_none.view(torch.int16).cpu())


# ---- at most 16 outlier columns: codes gathered once, in rows of 16 bytes ----
FEW = [
    # M, N, K, dtype, planted outlier columns, first columns (0 .. n-1) instead
    (257, 769, 448, BF16, 5, False),
    (72, 33, 576, F16, 16, False),
    (300, 700, 4096, F16, 6, False),   # few tiles: K split (tiles of 256 and of 224 columns)
    (96, 300, 512, F16, 4, True),      # columns 0 .. 3: the codes are CB's first columns
]


@pytest.mark.parametrize("fp8", [False, True], ids=["int8", "fp8"])
@pytest.mark.parametrize("M,N,K,dt,nout,prefix", FEW, ids=[f"{r[0]}x{r[1]}x{r[2]}-{r[4]}" for r in FEW])
def test_few_outlier_codes_gathered_match_direct(orc, M, N, K, dt, nout, prefix, fp8, tile_cols):
    """With at most 16 outlier columns the tiled product stages their weight
    codes from the table gathered once per call (by the activation kernel or
    by the product's own gather kernel) or, without a workspace, straight
    from CB per tile: the same bits either way, also after a call with more
    columns (a wider table) left the workspace stale, and against the oracle."""
    import torch
    import int8_quantized_matmul_row_amd as pkg
    from gpu_helpers import to_torch
    wl = synth.make_random(M, N, K, dt, seed=7 * M + N, n_outlier_cols=0 if prefix else nout, bias_sigma=0.01)
    if prefix:
        xb = synth.bits_to_f32(wl.X, dt)
        xb[:, :nout] = 20.0
        wl.X = synth.to_bits(xb, dt)
    dev = torch.device("cuda:0")
    X, W = to_torch(wl.X, dt, dev), to_torch(wl.W, dt, dev)
    bias = to_torch(wl.bias, dt, dev)
    qa, qw, mm, lin, lin_size = ((pkg.quantize_act_fp8, pkg.quantize_weight_fp8, pkg.matmul_fp8, pkg.linear_fp8,
                                  pkg.llmint8_linear_fp8_workspace_size) if fp8 else
                                 (pkg.quantize_act, pkg.quantize_weight, pkg.matmul, pkg.linear,
                                  pkg.llmint8_linear_workspace_size))
    CB, SCB = qw(W)
    q = qa(X, wl.threshold)
    n_out = int(q.n_out.item())
    log(f"[parity] few outlier codes {M}x{N}x{K} fp8={fp8} n_out={n_out} prefix={prefix} tile columns {tile_cols}")
    assert 1 <= n_out <= 16
    assert (pkg.outlier_columns(q).tolist() == list(range(n_out))) == prefix
    ref = mm(q, CB, SCB, bias=bias, workspace=(None, 0)).view(torch.int16).cpu()
    mm_bytes = pkg.llmint8_matmul_workspace_size(M, N, K)
    # a stale workspace: first a call with more than 16 columns (the wider layout)
    X_many = X.clone()
    X_many[:, 40:80] = 30.0
    q_many = qa(X_many, wl.threshold)
    assert int(q_many.n_out.item()) > 16
    ws = torch.full((mm_bytes,), 0x5A, dtype=torch.uint8, device=dev)
    mm(q_many, CB, SCB, bias=bias, workspace=(ws, mm_bytes))
    got = mm(q, CB, SCB, bias=bias, workspace=(ws, mm_bytes)).view(torch.int16).cpu()
    assert torch.equal(got, ref), "product's gather"
    base = lin_size(M, N, K)
    ws = torch.full((base,), 0x5A, dtype=torch.uint8, device=dev)
    lin(X_many, CB, SCB, bias=bias, threshold=wl.threshold, workspace=(ws, base))
    Y, q2 = lin(X, CB, SCB, bias=bias, threshold=wl.threshold, workspace=(ws, base))
    assert int(q2.n_out.item()) == n_out
    assert torch.equal(Y.view(torch.int16).cpu(), ref), "activation kernel's gather"
    # and the product against the oracle (the 1e-2 gate; the integer stages
    # are checked bit for bit by the other parity tests)
    r = (orc.forward_fp8 if fp8 else orc.forward)(wl.X, wl.W, dt, wl.threshold, bias=wl.bias)
    y = Y.float().cpu().numpy().astype(np.float64)
    assert np.abs(y - r["Y"]).max() <= 1e-2 * np.abs(r["Y"]).max()


# ---- K split over several workgroups per tile (few tiles, long K) -----------
SPLIT = [
    # M, N, K, dtype, planted outlier columns (tiles of 256 / 224 columns)
    (300, 700, 4096, F16, 40),    # 6 / 8 tiles, K split in 4; codes gathered too
    (80, 64, 57344, BF16, 3),     # 1 tile, split in 8
    (520, 300, 2048, BF16, 0),    # 6 tiles, split in 2; three tile rows
    (300, 700, 4160, F16, 20),    # split in 4; the last split ends in a half (64-byte) K stage
]


@pytest.mark.parametrize("fp8", [False, True], ids=["int8", "fp8"])
@pytest.mark.parametrize("M,N,K,dt,nout", SPLIT, ids=[f"{r[0]}x{r[1]}x{r[2]}" for r in SPLIT])
def test_split_k_matches_unsplit(M, N, K, dt, nout, fp8, tile_cols):
    """The split product (default workspace) against the unsplit one (no
    workspace): int8 accumulators and Y bit for bit; FP8 accumulators within
    fp32 reassociation error, Y within one 16-bit step.  Two split runs give
    the same bits."""
    import torch
    import int8_quantized_matmul_row_amd as pkg
    from gpu_helpers import to_torch
    wl = synth.make_random(M, N, K, dt, seed=7 * M + K, n_outlier_cols=nout, bias_sigma=0.01)
    dev = torch.device("cuda:0")
    X, W = to_torch(wl.X, dt, dev), to_torch(wl.W, dt, dev)
    bias = to_torch(wl.bias, dt, dev)
    if fp8:
        CB, SCB = pkg.quantize_weight_fp8(W)
        q = pkg.quantize_act_fp8(X, wl.threshold)
    else:
        CB, SCB = pkg.quantize_weight(W)
        q = pkg.quantize_act(X, wl.threshold)
    log(f"[parity] split K {M}x{N}x{K} fp8={fp8} n_out={int(q.n_out.item())} tile columns {tile_cols}")
    cdt = torch.float32 if fp8 else torch.int32

    def run(workspace):
        C = torch.empty((M, N), dtype=cdt, device=dev)
        if fp8:
            Y = pkg.matmul_fp8(q, CB, SCB, bias=bias, C_f32=C, workspace=workspace)
        else:
            Y = pkg.matmul(q, CB, SCB, bias=bias, C_i32=C, workspace=workspace)
        return Y.view(torch.int16).cpu(), C.cpu()

    Y0, C0 = run((None, 0))
    Y1, C1 = run(None)
    Y2, C2 = run(None)
    assert torch.equal(Y1, Y2) and torch.equal(C1, C2)
    # without the C export (more than 16 outlier columns: the other kernel)
    Y3 = (pkg.matmul_fp8 if fp8 else pkg.matmul)(q, CB, SCB, bias=bias).view(torch.int16).cpu()
    assert torch.equal(Y3, Y1)
    if not fp8:
        assert torch.equal(C1, C0)
        assert torch.equal(Y1, Y0)
    else:
        scale = C0.abs().max().item()
        assert (C1 - C0).abs().max().item() <= 1e-5 * scale
        # at most one 16-bit rounding step apart (plus a hair near zero)
        ft = torch.float16 if dt == F16 else torch.bfloat16
        y0, y1 = Y0.view(ft).float(), Y1.view(ft).float()
        step = 2.0 ** (-10 if dt == F16 else -7)
        assert ((y1 - y0).abs() <= step * y0.abs() + 1e-6 * y0.abs().max()).all()


# ---- outlier columns at the edges of the 128-byte K stages (the 224-column
# tile takes their weight codes from the B stages in its K loop; the 256-column
# tile gathers them from CB) --------------------------------------------------
EDGE = [
    # M, N, K, dtype, outlier columns
    (300, 448, 4160, F16, [0, 127, 128, 4095, 4096, 4159]),    # two in the last, half (64-byte) stage
    (300, 452, 4160, BF16, list(range(40, 56))),                # 16 adjacent columns in one stage; ragged N
    (80, 230, 192, F16, [63, 64, 65, 127, 128, 191] + [10 * i + 1 for i in range(11)]),  # 17: one past the 16
]


@pytest.mark.parametrize("M,N,K,dt,cols", EDGE, ids=[f"{r[0]}x{r[1]}x{r[2]}-{len(r[4])}" for r in EDGE])
def test_outlier_columns_at_stage_edges(orc, M, N, K, dt, cols, tile_cols):
    wl = synth.make_random(M, N, K, dt, seed=M + K, bias_sigma=0.01)
    x = synth.bits_to_f32(wl.X, dt)
    for j, c in enumerate(cols):
        x[(7 * j) % M, c] = 20.0 if j % 2 == 0 else -20.0
    wl.X = synth.to_bits(x, dt)
    g, ref = full_check(orc, wl, label=f"stage edges {M}x{N}x{K} tile columns {tile_cols}")
    assert list(ref["idx"]) == sorted(cols)


@pytest.mark.parametrize("M", [5, 48])
def test_threshold_boundary_and_zero_rows(orc, M):
    wl = synth.make_random(M, 70, 128, F16, seed=23)
    x = synth.bits_to_f32(wl.X, F16)
    x[:, 9] = 0.5
    x[M // 2, 9] = 6.0          # exactly the threshold: outlier column
    x[:, 100] = 0.25
    x[1, 100] = -5.99609375      # just below: stays int8
    x[2] = 0.0                   # an all-zero row
    x[3, :] = 0.0
    x[3, 9] = 6.0                # a row whose only mass is in an outlier column
    wl.X = synth.f32_to_f16_bits(x)
    w = synth.bits_to_f32(wl.W, F16)
    w[5] = 0.0                   # an all-zero weight row
    wl.W = synth.f32_to_f16_bits(w)
    g, ref = full_check(orc, wl, label=f"boundary M={M}")
    assert 9 in list(ref["idx"]) and 100 not in list(ref["idx"])
    assert g["SCA"][2] == 0 and g["SCA"][3] == 0 and g["SCB"][5] == 0


def test_empty_batch_sets_zero_outliers():
    import torch
    import int8_quantized_matmul_row_amd as pkg
    dev = torch.device("cuda:0")
    X = torch.empty((0, 128), dtype=torch.float16, device=dev)
    q = pkg.alloc_act(0, 128, torch.float16, dev)
    q.n_out.fill_(-7)
    pkg.quantize_act(X, 6.0, out=q)
    W = torch.randn((32, 128), dtype=torch.float16, device=dev)
    CB, SCB = pkg.quantize_weight(W)
    Y = pkg.matmul(q, CB, SCB)
    torch.cuda.synchronize()
    assert int(q.n_out.item()) == 0 and Y.shape == (0, 32)


def test_deterministic_and_bias_applied(orc):
    import torch
    wl = synth.make_random(300, 520, 320, F16, seed=31, n_outlier_cols=3, bias_sigma=0.01)
    a = run_gpu(wl)
    b = run_gpu(wl, weight=a["weight"])
    assert np.array_equal(a["Y"], b["Y"])
    assert torch.equal(a["C_dev"], b["C_dev"])
    nb = synth.Workload(**{**wl.__dict__, "bias": None})
    c = run_gpu(nb, weight=a["weight"])
    diff = synth.bits_to_f32(a["Y"], F16).astype(np.float64) - synth.bits_to_f32(c["Y"], F16)
    bias = synth.bits_to_f32(wl.bias, F16).astype(np.float64)
    # Y(bias) - Y(no bias) equals the bias up to two fp16 output roundings
    assert np.abs(diff - bias[None, :]).max() <= 2 * 2.0 ** -11 * 8


# ---- full-size workloads on sampled rows ------------------------------------
def sampled_check(orc, wl, n_rows, threshold=None, weight_cache=None, label=None):
    """Every quantization stage in full; C and Y on n_rows sampled rows (rows 0
    and M-1 among them), or on every row when n_rows >= M."""
    t = wl.threshold if threshold is None else threshold
    label = label or f"{wl.name} t={t}"
    every = n_rows >= wl.M
    log(f"[parity] {label} M={wl.M} N={wl.N} K={wl.K} "
        f"{'every row' if every else f'sampled rows={n_rows}'} (oracle on {host_threads()} threads)")
    rows = None if every else sample_rows(wl.M, n_rows)
    if weight_cache is not None and wl.name in weight_cache:
        (CB_ref, SCB_ref), dev_w = weight_cache[wl.name]
        g = run_gpu(wl, t, weight=dev_w)
    else:
        g = run_gpu(wl, t)
        CB_ref, SCB_ref = orc.quantize_weight(wl.W, wl.dtype)
        assert np.array_equal(g["CB"], CB_ref), f"{label}: CB"
        assert np.array_equal(g["SCB"], SCB_ref), f"{label}: SCB"
        if weight_cache is not None:
            weight_cache[wl.name] = ((CB_ref, SCB_ref), g["weight"])
    ref = oracle_forward(orc, wl, t, (CB_ref, SCB_ref), rows=rows)
    err, scale = compare(wl, g, ref, rows=rows, label=label)
    log(f"[parity] {label}: ok, n_out={g['n_out']} max|dY|={err:.3g} max|Y|={scale:.3g}")
    return g


def test_prefill_full_size(orc):
    """2048 x 16384 x 4096: C and Y on every row."""
    wl = synth.make_workload("prefill")
    sampled_check(orc, wl, wl.M)


@pytest.fixture(scope="module")
def sweep_weight():
    return {}


@pytest.mark.parametrize("name", ["sweep_0", "sweep_0.1", "sweep_1", "sweep_5"])
def test_sweep_full_size(orc, name, sweep_weight):
    wl = synth.make_workload(name, with_weight=not sweep_weight)
    wl.name = "sweep"  # one weight for the four densities
    sampled_check(orc, wl, 64, weight_cache=sweep_weight, label=name)


@pytest.mark.parametrize("t", [float("inf"), 0.0])
def test_sweep_threshold_extremes_full_size(orc, t, sweep_weight):
    wl = synth.make_workload("sweep_0.1", with_weight=not sweep_weight)
    wl.name = "sweep"
    g = sampled_check(orc, wl, 16 if t == 0.0 else 64, threshold=t, weight_cache=sweep_weight,
                      label=f"sweep_0.1 t={t}")
    assert g["n_out"] == (0 if t != 0.0 else wl.K)


@pytest.mark.parametrize("name", ["bloom_up", "bloom_down"])
def test_bloom_ffn_full_size(orc, name):
    wl = synth.make_workload(name)
    sampled_check(orc, wl, 48)


# batched decode at real layer sizes through the weight-streaming product:
# workgroups of 64 channels with four, two and one groups of 16 rows
# (64 x 16384 x 16384, 24 x 28672 x 8192, 16 x 28672 x 8192), workgroups of
# 16 channels (32 x 8192 x 28672); every row
@pytest.mark.parametrize("M,N,K,dt,nout", [(64, 16384, 16384, F16, 6), (24, 28672, 8192, F16, 40),
                                           (32, 8192, 28672, BF16, 3), (16, 28672, 8192, BF16, 4)])
def test_batched_decode_streaming_full_size(orc, M, N, K, dt, nout):
    wl = synth.make_random(M, N, K, dt, seed=M + 7, n_outlier_cols=nout, bias_sigma=0.01)
    sampled_check(orc, wl, M)


# ---- the one-call forward (llmint8_linear): fused small-M kernel and the
# ---- quantize_act + matmul sequence, every stage against the oracle ----------
from gpu_helpers import run_gpu_linear  # noqa: E402

LINEAR = [
    # M, N, K, dtype, planted outlier columns, bias, threshold
    (8, 4096, 4096, F16, 4, False, 6.0),      # the decode workload's shape
    (1, 100, 64, F16, 0, True, 6.0),
    (5, 333, 1024, BF16, 3, True, 6.0),
    (16, 1030, 4096, F16, 6, True, 6.0),      # largest fused M at K = 4096
    (8, 520, 8192, BF16, 9, False, 6.0),      # largest fused K at M = 8
    (12, 260, 2048, F16, 12, True, 0.0),      # every column an outlier
    (7, 96, 512, F16, 2, True, float("inf")),
    (16, 64, 8192, F16, 2, False, 6.0),       # M*K beyond the fused bound
    (65, 300, 640, BF16, 3, True, 6.0),       # tiled path through llmint8_linear
    (33, 300, 640, BF16, 3, True, 6.0),       # the streaming kernel through llmint8_linear
    (8, 200, 4160, F16, 3, True, 6.0),        # last K slice one step deep
    (3, 64, 192, BF16, 1, False, 6.0),        # one slice, a wave with no step
    (16, 77, 2112, BF16, 2, True, 2.5),       # ~90 outlier columns per slice
    (8, 4096, 1024, F16, 1, True, 6.0),       # four slices of 256 columns
    (257, 769, 448, BF16, 40, True, 6.0),     # tiled; the activation kernel gathers codes
    (72, 33, 576, F16, 150, True, 6.0),
    (300, 100, 1024, F16, 2, True, 0.0),      # more outlier columns than the workspace holds
    # the fused decode kernel with more than 8 outlier columns: the 16-bit
    # product as MFMAs over all of K against X masked to the outlier columns
    (8, 512, 4096, F16, 4, True, 0.0),
    (4, 300, 8192, BF16, 40, False, 6.0),     # two chunks per thread
    (8, 96, 4096, BF16, 0, True, 2.0),        # a few hundred columns at t = 2
]


@pytest.mark.parametrize("M,N,K,dt,nout,bias,t", LINEAR,
                         ids=[f"{r[0]}x{r[1]}x{r[2]}-{synth.DTYPE_NAMES[r[3]]}-t{r[6]}"
                              for r in LINEAR])
def test_linear_one_call(orc, M, N, K, dt, nout, bias, t):
    wl = synth.make_random(M, N, K, dt, seed=3 * M + N + K, n_outlier_cols=nout,
                           bias_sigma=0.01 if bias else None)
    label = f"linear {M}x{N}x{K} t={t}"
    log(f"[parity] {label}")
    g = run_gpu_linear(wl, t)
    ref = orc.forward(wl.X, wl.W, wl.dtype, t, bias=wl.bias)
    err, scale = compare(wl, g, ref, label=label)
    log(f"[parity] {label}: ok, n_out={g['n_out']} max|dY|={err:.3g}")


def test_linear_decode_workload_matches_two_calls(orc):
    """The fused forward and quantize_act + matmul give identical integer stages
    on the decode workload, and both match the oracle."""
    wl = synth.make_workload("decode")
    a = run_gpu_linear(wl)
    b = run_gpu(wl, weight=a["weight"])
    for key in ("CA", "SCA", "idx", "XO"):
        assert np.array_equal(a[key], b[key]), key
    import torch
    assert torch.equal(a["C_dev"], b["C_dev"])
    ref = orc.forward(wl.X, wl.W, wl.dtype, wl.threshold)
    compare(wl, a, {**ref, "CB": a["weight"][0].cpu().numpy(),
                    "SCB": a["weight"][1].cpu().numpy()}, label="linear decode")


def test_linear_workspace_reuse_any_shape(orc):
    """One workspace, sized for the largest call, serves fused and unfused
    calls of different shapes in turn."""
    import torch
    import int8_quantized_matmul_row_amd as pkg
    dev = torch.device("cuda:0")
    shapes = [(8, 4096, 4096, F16), (33, 300, 640, BF16), (16, 1030, 4096, F16),
              (5, 333, 1024, BF16), (8, 4096, 4096, F16)]
    size = max(pkg.llmint8_linear_workspace_size(M, N, K) for M, N, K, _ in shapes)
    ws = (torch.empty((max(size, 1),), dtype=torch.uint8, device=dev), size)
    for i, (M, N, K, dt) in enumerate(shapes):
        wl = synth.make_random(M, N, K, dt, seed=100 + i, n_outlier_cols=3, bias_sigma=0.01)
        log(f"[parity] workspace reuse {M}x{N}x{K}")
        g = run_gpu_linear(wl, workspace=ws)
        ref = orc.forward(wl.X, wl.W, wl.dtype, wl.threshold, bias=wl.bias)
        compare(wl, g, ref, label=f"reuse {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K,nout", [(40, 64, 57344, 3), (300, 700, 4096, 40)],
                         ids=["split-K", "gathered-codes"])
def test_tiled_product_graph_replays(M, N, K, nout):
    """The tiled product with its workspace (split-K counters zeroed by a
    kernel, outlier codes gathered): replays of a captured HIP graph, with
    eager work and a call on other inputs between them, match the eager
    result bit for bit, both for llmint8_matmul and for llmint8_linear."""
    import torch
    import int8_quantized_matmul_row_amd as pkg
    from gpu_helpers import to_torch
    dev = torch.device("cuda:0")
    wl = synth.make_random(M, N, K, BF16, seed=M + K, n_outlier_cols=nout, bias_sigma=0.01)
    X, W = to_torch(wl.X, BF16, dev), to_torch(wl.W, BF16, dev)
    bias = to_torch(wl.bias, BF16, dev)
    X2 = (X * 0.5).contiguous()
    CB, SCB = pkg.quantize_weight(W)
    log(f"[parity] graph replays of the tiled product {M}x{N}x{K}")
    q = pkg.alloc_act(M, K, torch.bfloat16, dev)
    q2 = pkg.alloc_act(M, K, torch.bfloat16, dev)
    mws = pkg.matmul_workspace(M, N, K, dev)
    lws = pkg.linear_workspace(M, N, K, dev)
    Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    C = torch.empty((M, N), dtype=torch.int32, device=dev)
    stream = torch.cuda.Stream()

    def product():
        pkg.quantize_act(X, wl.threshold, out=q, stream=stream)
        pkg.matmul(q, CB, SCB, bias=bias, out=Y, C_i32=C, workspace=mws, stream=stream)

    def forward():
        pkg.linear(X, CB, SCB, bias=bias, threshold=wl.threshold, out=Y, act=q, C_i32=C,
                   workspace=lws, stream=stream)

    for fn in (product, forward):
        with torch.cuda.stream(stream):
            fn()
        torch.cuda.synchronize()
        Y0, C0 = Y.clone(), C.clone()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            fn()
        for r in range(4):
            Y.zero_()
            C.zero_()
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            assert torch.equal(Y, Y0), f"{fn.__name__} replay {r}: Y differs"
            assert torch.equal(C, C0), f"{fn.__name__} replay {r}: C differs"
            # other inputs through the same workspace, eagerly, between replays
            pkg.quantize_act(X2, wl.threshold, out=q2)
            pkg.matmul(q2, CB, SCB, workspace=mws)
            pkg.linear(X2, CB, SCB, threshold=wl.threshold, workspace=lws)
            torch.cuda.synchronize()


def test_linear_fused_repeatable_and_graph_replays():
    """The fused forward gives the same bits on every call, and replays of a
    captured HIP graph (with eager work between them) match the eager call."""
    import torch
    import int8_quantized_matmul_row_amd as pkg
    dev = torch.device("cuda:0")
    wl = synth.make_workload("decode")
    X = torch.from_numpy(wl.X.view(np.int16)).to(dev).view(torch.float16)
    W = torch.from_numpy(wl.W.view(np.int16)).to(dev).view(torch.float16)
    CB, SCB = pkg.quantize_weight(W)
    ws = pkg.linear_workspace(wl.M, wl.N, wl.K, dev)
    q = pkg.alloc_act(wl.M, wl.K, torch.float16, dev)
    Y = torch.empty((wl.M, wl.N), dtype=torch.float16, device=dev)
    C = torch.empty((wl.M, wl.N), dtype=torch.int32, device=dev)
    pkg.linear(X, CB, SCB, threshold=wl.threshold, out=Y, act=q, C_i32=C, workspace=ws)
    torch.cuda.synchronize()
    Y0, C0 = Y.clone(), C.clone()
    for _ in range(3):
        Y.zero_()
        pkg.linear(X, CB, SCB, threshold=wl.threshold, out=Y, act=q, C_i32=C, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(Y, Y0) and torch.equal(C, C0)
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        pkg.linear(X, CB, SCB, threshold=wl.threshold, out=Y, act=q, C_i32=C, workspace=ws,
                   stream=stream)
    for r in range(4):
        Y.zero_()
        C.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(Y, Y0), f"graph replay {r}: Y differs"
        assert torch.equal(C, C0), f"graph replay {r}: C differs"
        _ = (X.float() * 2).sum().item()  # unrelated eager work between replays
