"""GPU parity on seeded random shapes: every stage against the oracle, through
both calls the product has.

* quantize_act + matmul with the int32 accumulators exported: CB, SCB, CA,
  SCA, the outlier list, XO and C bit for bit, Y within the gate;
* the one-call forward (llmint8_linear) with its default workspace and no
  export: the activation kernel's gather of the outlier codes (in rows of 16
  bytes up to 16 columns, of the workspace's width past them), the tiled
  product's reads of that table and, past 16 columns, its outlier K loop.

The shapes cover tokens from just past the small-M kernels to several tile
rows, ragged N, K from one 64-byte unit to dozens of stages, both 16-bit
types and outlier counts around the 16-column limits, under both tile widths.
"""
import numpy as np
import pytest

import synth
from gpu_helpers import check_y, compare, log, run_gpu, to_torch

pytestmark = pytest.mark.gpu


def _cases(n=24, seed=2026):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        while True:
            M = int(np.exp(rng.uniform(np.log(17), np.log(700))))
            N = int(rng.integers(1, 900))
            K = 64 * int(rng.integers(1, 48))
            if M * N * K <= 2e8:
                break
        dt = synth.F16 if rng.random() < 0.5 else synth.BF16
        nout = int(rng.choice([0, 1, 2, 3, 5, 8, 13, 16, 17, 24, 40]))
        nout = min(nout, K // 2)
        out.append((M, N, K, dt, nout, bool(rng.random() < 0.5), 1000 + i))
    return out


CASES = _cases()


@pytest.fixture(scope="module", autouse=True)
def gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import int8_quantized_matmul_row_amd as pkg
    pkg.lib()


@pytest.fixture(params=["256", "224"], ids=["w256", "w224"])
def tile_cols(request, monkeypatch):
    monkeypatch.setenv("LLMINT8_TILE_COLS", request.param)
    return int(request.param)


@pytest.mark.parametrize("M,N,K,dt,nout,with_bias,seed", CASES,
                         ids=[f"{c[0]}x{c[1]}x{c[2]}-{synth.DTYPE_NAMES[c[3]]}-{c[4]}" for c in CASES])
def test_random_shape_both_calls(orc, M, N, K, dt, nout, with_bias, seed, tile_cols):
    import torch
    import int8_quantized_matmul_row_amd as pkg
    wl = synth.make_random(M, N, K, dt, seed=seed, n_outlier_cols=nout, bias_sigma=0.01 if with_bias else None)
    label = f"random {M}x{N}x{K} {synth.DTYPE_NAMES[dt]} planted {nout} tile columns {tile_cols}"
    log(f"[parity] {label}")
    ref = orc.forward(wl.X, wl.W, wl.dtype, wl.threshold, bias=wl.bias)
    g = run_gpu(wl)
    compare(wl, g, ref, label=label + " (matmul)")
    dev = torch.device("cuda:0")
    X = to_torch(wl.X, dt, dev)
    bias = None if wl.bias is None else to_torch(wl.bias, dt, dev)
    CB, SCB = g["weight"]
    Y, q = pkg.linear(X, CB, SCB, bias=bias, threshold=wl.threshold)
    torch.cuda.synchronize()
    n_out = int(q.n_out.item())
    assert n_out == len(ref["idx"])
    assert np.array_equal(q.idx[:n_out].cpu().numpy(), ref["idx"])
    assert np.array_equal(q.CA.cpu().numpy(), ref["CA"])
    assert np.array_equal(q.SCA.cpu().numpy(), ref["SCA"])
    check_y(Y.view(torch.int16).cpu().numpy().view(np.uint16), ref["Y"], dt, label + " (linear)")
