"""The C-ABI library on the CPU: it loads, exports what the header declares,
and rejects bad arguments before making any HIP call (no GPU needed)."""
import ctypes
import os
import re

import pytest

import int8_quantized_matmul_row_amd as pkg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "llmint8.h")

OK, INVALID, UNSUPPORTED = 0, 1, 2
A = 0x10000  # a 16-byte aligned fake address; never dereferenced by these tests


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:[\w\s\*]+?)\b(llmint8_\w+)\s*\(", text, re.M)))


def test_library_loads_and_exports_every_declared_symbol():
    lib = pkg.lib()
    names = declared_functions()
    assert set(names) == set(pkg.EXPORTS), names
    for name in names:
        assert getattr(lib, name) is not None


def test_status_strings():
    for s, text in pkg.STATUS.items():
        assert pkg.llmint8_status_string(s) == text
    assert pkg.llmint8_status_string(99) == "unknown status"
    assert pkg.llmint8_last_hip_error() == 0


def qw(W=A, dtype=0, N=8, K=64, CB=A, SCB=A):
    return pkg.lib().llmint8_quantize_weight(W, dtype, N, K, CB, SCB, None)


def test_quantize_weight_validation():
    assert qw(dtype=2) == INVALID
    assert qw(N=-1) == INVALID
    assert qw(K=-64) == INVALID
    assert qw(K=0) == UNSUPPORTED
    assert qw(K=100) == UNSUPPORTED
    assert qw(K=pkg.K_MAX + 64) == UNSUPPORTED
    assert qw(N=1 << 31) == UNSUPPORTED
    assert qw(W=None) == INVALID
    assert qw(CB=None) == INVALID
    assert qw(SCB=A + 4) == INVALID      # misaligned
    assert qw(N=0, W=None, CB=None, SCB=None) == OK   # empty: nothing to do


def qa(X=A, dtype=0, M=64, K=512, t=6.0, CA=A, SCA=A, idx=A, n=A, XO=A, ws=A, wsb=1 << 30):
    return pkg.lib().llmint8_quantize_act(X, dtype, M, K, ctypes.c_float(t), CA, SCA, idx, n, XO,
                                          ws, wsb, None)


def test_quantize_act_validation():
    assert qa(t=float("nan")) == INVALID
    assert qa(t=-1.0) == INVALID
    assert qa(dtype=-1) == INVALID
    assert qa(K=96) == UNSUPPORTED
    assert qa(M=-1) == INVALID
    assert qa(n=None) == INVALID
    assert qa(X=None) == INVALID
    assert qa(XO=A + 2) == INVALID
    need = pkg.llmint8_quantize_act_workspace_size(64, 512)
    assert need > 0
    assert qa(ws=None) == INVALID
    assert qa(wsb=need - 1) == INVALID


def test_tile_width_override(monkeypatch):
    # LLMINT8_TILE_COLS forces the tiled product's tile width; the workspace
    # size follows it (112 tiles of 256 columns, split in 2)
    monkeypatch.setenv("LLMINT8_TILE_COLS", "256")
    assert pkg.llmint8_matmul_workspace_size(512, 14336, 57344) == \
        512 + 2 * 112 * (256 * 256 * 4) + 14336 * 1024
    monkeypatch.setenv("LLMINT8_TILE_COLS", "224")
    assert pkg.llmint8_matmul_workspace_size(2048, 16384, 4096) == 16 << 20  # no split either way
    assert pkg.llmint8_matmul_workspace_size(65, 4096, 4096) == \
        256 + 4 * 19 * (256 * 224 * 4) + 4096 * 1024
    monkeypatch.setenv("LLMINT8_TILE_COLS", "other")  # ignored
    assert pkg.llmint8_matmul_workspace_size(512, 14336, 57344) == \
        512 + 2 * 128 * (256 * 224 * 4) + 14336 * 1024


def test_workspace_sizes():
    assert pkg.llmint8_quantize_act_workspace_size(8, 4096) == 0      # one-launch path
    assert pkg.llmint8_quantize_act_workspace_size(2048, 4096) > 0
    assert pkg.llmint8_quantize_act_workspace_size(64, 100) == 0       # unsupported K
    # the tiled product: split-K partial tiles when the 256 x W tiles fill
    # under half of the 256 CUs (256 * W * 4 bytes each, per split, after 256
    # bytes of counters), then the gathered outlier codes (one byte per weight
    # row and column, up to 1024 columns, fewer when K is smaller); nothing
    # for the small-M kernel.  W = 224 where it takes fewer MFMA cycles per CU
    # (one round of workgroups either way: 224 columns each), else 256.
    P224, P256 = 256 * 224 * 4, 256 * 256 * 4
    assert pkg.llmint8_matmul_workspace_size(8, 4096, 4096) == 0
    assert pkg.llmint8_matmul_workspace_size(16, 4096, 4096) == 0
    assert pkg.llmint8_matmul_workspace_size(64, 4096, 4096) == 0   # up to 64 rows: the streaming kernel
    # W = 224: 19 tiles, K = 32 stages split in 4
    assert pkg.llmint8_matmul_workspace_size(65, 4096, 4096) == \
        256 + 4 * 19 * P224 + 4096 * 1024
    # W = 256: 512 tiles (2 rounds; 592 tiles of 224 take 3): no split
    assert pkg.llmint8_matmul_workspace_size(2048, 16384, 4096) == 16 << 20
    # 2 tiles, but K is 1 stage: no split
    assert pkg.llmint8_matmul_workspace_size(300, 33, 128) == 33 * 128
    # 1 tile, split in 8 (the most)
    assert pkg.llmint8_matmul_workspace_size(80, 64, 57344) == \
        256 + 8 * P224 + 64 * 1024
    # the BLOOM-shaped down projection: 128 tiles of 224 columns (112 of 256
    # would leave 32 CUs idle), split in 2
    assert pkg.llmint8_matmul_workspace_size(512, 14336, 57344) == \
        512 + 2 * 128 * P224 + 14336 * 1024
    assert pkg.llmint8_matmul_workspace_size(300, 33, 96) == 0           # unsupported K
    assert pkg.llmint8_matmul_workspace_size(300, 0, 4096) == 0          # empty: no tiles
    assert pkg.llmint8_linear_workspace_size(300, 0, 4096) == \
        pkg.llmint8_quantize_act_workspace_size(300, 4096)
    assert pkg.llmint8_linear_workspace_size(2048, 16384, 4096) >= \
        pkg.llmint8_quantize_act_workspace_size(2048, 4096) + (16 << 20)


def mm(dtype=0, M=32, N=64, K=128, CA=A, SCA=A, idx=A, n=A, XO=A, CB=A, SCB=A, bias=None, Y=A,
       C=None, ws=None, wsb=0):
    return pkg.lib().llmint8_matmul(dtype, M, N, K, CA, SCA, idx, n, XO, CB, SCB, bias, Y, C, ws,
                                    wsb, None)


def test_matmul_validation():
    assert mm(dtype=3) == INVALID
    assert mm(K=65) == UNSUPPORTED
    assert mm(K=0) == UNSUPPORTED
    assert mm(N=-5) == INVALID
    for key in ("CA", "SCA", "idx", "n", "XO", "CB", "SCB", "Y"):
        assert mm(**{key: None}) == INVALID, key
    assert mm(bias=A + 2) == INVALID
    assert mm(C=A + 8) == INVALID
    assert mm(M=0, CA=None, SCA=None, XO=None, Y=None) == OK
    assert mm(N=0, CB=None, SCB=None, Y=None) == OK


def test_binding_refuses_cpu_tensors():
    torch = pytest.importorskip("torch")
    with pytest.raises(ValueError):
        pkg.quantize_weight(torch.zeros((4, 64), dtype=torch.float16))


def test_fp8_entry_points_validation():
    L = pkg.lib()
    assert L.llmint8_quantize_weight_fp8(A, 0, 8, 100, A, A, None) == UNSUPPORTED
    assert L.llmint8_quantize_weight_fp8(None, 0, 8, 64, A, A, None) == INVALID
    assert L.llmint8_quantize_weight_fp8(None, 0, 0, 64, None, None, None) == OK
    assert L.llmint8_quantize_act_fp8(A, 0, 64, 512, ctypes.c_float(float("nan")), A, A, A, A, A,
                                      A, 1 << 30, None) == INVALID
    assert L.llmint8_quantize_act_fp8(A, 0, 64, 512, ctypes.c_float(6.0), A, A, A, A, A, None, 0,
                                      None) == INVALID          # workspace required
    args = [0, 32, 64, 128, A, A, A, A, A, A, A, None, A, None, None, 0, None]
    for i in (4, 5, 6, 7, 8, 9, 10, 12):                        # required pointers
        bad = list(args)
        bad[i] = None
        assert L.llmint8_matmul_fp8(*bad) == INVALID, i
    bad = list(args)
    bad[13] = A + 4                                             # misaligned C_f32
    assert L.llmint8_matmul_fp8(*bad) == INVALID
    # the FP8 forward has no fused small-M kernel, so it needs the act workspace
    assert pkg.llmint8_linear_fp8_workspace_size(2048, 4096, 4096) >= \
        pkg.llmint8_quantize_act_workspace_size(2048, 4096) > 0
    assert pkg.llmint8_linear_fp8_workspace_size(8, 4096, 4096) == 0
    assert pkg.llmint8_linear_fp8_workspace_size(8, 4096, 100) == 0


def test_peak_mfma_rejects_bad_arguments_before_any_hip_call():
    L = pkg.lib()
    ok = dict(fp8=0, operands=A, operand_bytes=262144, sink=A, sink_bytes=1024 * 4, blocks=4, iters=1)

    def call(**kw):
        a = {**ok, **kw}
        return L.llmint8_peak_mfma(a["fp8"], a["operands"], a["operand_bytes"], a["sink"],
                                   a["sink_bytes"], a["blocks"], a["iters"], None)

    assert call(fp8=2) == INVALID
    assert call(operands=None) == INVALID
    assert call(operands=A + 4) == INVALID          # misaligned
    assert call(sink=None) == INVALID
    assert call(operand_bytes=262143) == INVALID
    assert call(sink_bytes=4 * 1024 - 1) == INVALID  # one word per thread of 4 blocks
    assert call(blocks=0) == INVALID
    assert call(iters=0) == INVALID


def test_noalloc_refuses_what_its_scratch_cannot_hold_before_any_hip_call():
    """llmint8_linear_noalloc: the same argument checks as llmint8_linear, and
    shapes whose workspace exceeds the static scratch array are refused."""
    L = pkg.lib()

    def call(M=2048, N=16384, K=4096, t=6.0, X=A, CB=A, SCB=A, Y=A, CA=A, SCA=A, idx=A, n=A, XO=A):
        return L.llmint8_linear_noalloc(X, 0, M, N, K, ctypes.c_float(t), CB, SCB, None, Y, CA, SCA,
                                        idx, n, XO, None, None)

    assert pkg.llmint8_linear_workspace_size(4096, 28672, 8192) <= pkg.SCRATCH_BYTES
    assert pkg.llmint8_linear_workspace_size(512, 14336, 57344) > pkg.SCRATCH_BYTES
    assert call(M=512, N=14336, K=57344) == UNSUPPORTED
    assert call(K=100) == UNSUPPORTED
    assert call(t=float("nan")) == INVALID
    assert call(t=-1.0) == INVALID
    for key in ("X", "CB", "SCB", "Y", "CA", "SCA", "idx", "n", "XO"):
        assert call(**{key: None}) == INVALID, key
    assert call(XO=A + 2) == INVALID
