"""llmint8_linear_noalloc, the forward for callers that cannot allocate device
memory, against llmint8_linear with a workspace of its own: two calls in a row
through the C ABI, the second smaller, each with split-K partial tiles and more
than 16 outlier columns (so the static scratch holds the activation kernel's
partial masks, the split-K counters and partial tiles, and the gathered weight
codes).  Every output must be identical; both are also checked against the
oracle."""
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


def outputs(M, N, K, dtype_t, dev):
    import torch
    return dict(Y=torch.empty((M, N), dtype=dtype_t, device=dev),
                CA=torch.empty((M, K), dtype=torch.int8, device=dev),
                SCA=torch.empty((M,), dtype=torch.float32, device=dev),
                idx=torch.empty((K,), dtype=torch.int32, device=dev),
                n_out=torch.empty((1,), dtype=torch.int32, device=dev),
                XO=torch.empty((M * K,), dtype=dtype_t, device=dev),
                C=torch.empty((M, N), dtype=torch.int32, device=dev))


def call(noalloc, wl, X, CB, SCB, bias, o, stream):
    import int8_quantized_matmul_row_amd as pkg
    args = (X.data_ptr(), wl.dtype, wl.M, wl.N, wl.K, wl.threshold, CB.data_ptr(), SCB.data_ptr(),
            None if bias is None else bias.data_ptr(), o["Y"].data_ptr(), o["CA"].data_ptr(),
            o["SCA"].data_ptr(), o["idx"].data_ptr(), o["n_out"].data_ptr(), o["XO"].data_ptr(),
            o["C"].data_ptr())
    if noalloc:
        pkg.llmint8_linear_noalloc(*args, stream)
    else:
        ws, nbytes = pkg.linear_workspace(wl.M, wl.N, wl.K, X.device)
        pkg.llmint8_linear(*args, ws.data_ptr(), nbytes, stream)
        return ws


CASES = [
    # M, N, K, dtype, outlier columns: all split K in 2 (few tiles, K = 2048);
    # the last holds at most 16 outlier columns (their codes gathered in rows
    # of 16 bytes, after a call that left the wider layout in the scratch)
    (512, 1536, 2048, synth.F16, 40),
    (260, 700, 2048, synth.BF16, 20),
    (260, 700, 2048, synth.F16, 6),
]


def test_noalloc_matches_linear_twice_in_a_row(orc):
    import torch
    import int8_quantized_matmul_row_amd as pkg
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream().cuda_stream
    for i, (M, N, K, dt, n_cols) in enumerate(CASES):
        wl = synth.make_random(M, N, K, dt, seed=31 + i, n_outlier_cols=n_cols, bias_sigma=0.01)
        assert pkg.llmint8_linear_workspace_size(M, N, K) <= pkg.SCRATCH_BYTES
        log(f"[noalloc] call {i + 1}: {M}x{N}x{K} {synth.DTYPE_NAMES[dt]}, {n_cols} outlier columns")
        dtype_t = torch.float16 if dt == synth.F16 else torch.bfloat16
        X = to_torch(wl.X, dt, dev)
        CB, SCB = pkg.quantize_weight(to_torch(wl.W, dt, dev))
        bias = to_torch(wl.bias, dt, dev)
        ref_o, got_o = outputs(M, N, K, dtype_t, dev), outputs(M, N, K, dtype_t, dev)
        ws = call(False, wl, X, CB, SCB, bias, ref_o, stream)
        call(True, wl, X, CB, SCB, bias, got_o, stream)
        torch.cuda.synchronize()
        del ws
        n_out = int(got_o["n_out"].item())
        assert n_out == int(ref_o["n_out"].item()) == n_cols
        n_pad = (n_out + 31) // 32 * 32
        for k in ("CA", "SCA", "C"):
            assert torch.equal(got_o[k], ref_o[k]), k
        assert torch.equal(got_o["idx"][:n_out], ref_o["idx"][:n_out])
        assert torch.equal(got_o["XO"][:M * n_pad].view(torch.int16), ref_o["XO"][:M * n_pad].view(torch.int16))
        assert torch.equal(got_o["Y"].view(torch.int16), ref_o["Y"].view(torch.int16)), "Y bits"
        ref = orc.forward(wl.X, wl.W, dt, wl.threshold, bias=wl.bias)
        assert np.array_equal(got_o["C"].cpu().numpy(), ref["C"])
        check_y(bits_of(got_o["Y"]), ref["Y"], dt, f"noalloc call {i + 1}")
