"""Linear8bitLt on the GPU: quantize once on placement, forward against the
CPU oracle, model conversion, the chained FFN block (up -> GeLU -> down) and
the checkpoint round trip.

"A Gentle Introduction to 8-bit Matrix Multiplication for transformers at
scale", section "Usage"."""
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


def make_layer(wl):
    import torch
    from int8_quantized_matmul_row_amd import nn as n8
    lin = torch.nn.Linear(wl.K, wl.N, bias=wl.bias is not None,
                          dtype=torch.float16 if wl.dtype == synth.F16 else torch.bfloat16)
    with torch.no_grad():
        lin.weight.copy_(to_torch(wl.W, wl.dtype, "cpu"))
        if wl.bias is not None:
            lin.bias.copy_(to_torch(wl.bias, wl.dtype, "cpu"))
    return n8.Linear8bitLt.from_linear(lin, threshold=wl.threshold)


@pytest.mark.parametrize("M,N,K,dt", [(8, 512, 1024, synth.F16), (40, 300, 640, synth.BF16)])
def test_layer_forward_matches_oracle(orc, M, N, K, dt):
    import torch
    wl = synth.make_random(M, N, K, dt, seed=77 + M, n_outlier_cols=3, bias_sigma=0.01)
    log(f"[nn] Linear8bitLt {M}x{N}x{K}")
    m = make_layer(wl).cuda()
    assert m.quantized and m.weight is None
    ref = orc.forward(wl.X, wl.W, wl.dtype, wl.threshold, bias=wl.bias)
    assert np.array_equal(m.CB.cpu().numpy(), ref["CB"])
    assert np.array_equal(m.SCB.cpu().numpy(), ref["SCB"])
    x = to_torch(wl.X, wl.dtype, "cuda").reshape(2, M // 2, K) if M % 2 == 0 else \
        to_torch(wl.X, wl.dtype, "cuda")
    y = m(x)
    torch.cuda.synchronize()
    assert y.shape == (*x.shape[:-1], N)
    assert int(m.last_outlier_count.item()) == len(ref["idx"])
    check_y(bits_of(y.reshape(M, N)), ref["Y"], wl.dtype, "Linear8bitLt")


def test_placing_again_does_not_requantize(orc):
    import torch
    wl = synth.make_random(4, 64, 128, synth.F16, seed=3, n_outlier_cols=1, bias_sigma=0.01)
    m = make_layer(wl).cuda()
    cb_ptr, scb = m.CB.data_ptr(), m.SCB.clone()
    m = m.cuda().to("cuda:0").half()
    assert m.CB.data_ptr() == cb_ptr and m.CB.dtype == torch.int8
    assert m.SCB.dtype == torch.float32 and torch.equal(m.SCB, scb)
    # the forward after the casts still reads fp32 scales
    y = m(to_torch(wl.X, wl.dtype, "cuda"))
    torch.cuda.synchronize()
    ref = orc.forward(wl.X, wl.W, wl.dtype, wl.threshold, bias=wl.bias)
    check_y(bits_of(y), ref["Y"], wl.dtype, "forward after .half()")


def test_cast_to_bf16_switches_the_layer_dtype(orc):
    """A float16 layer cast to bfloat16 keeps CB and SCB and takes bf16 input;
    the oracle sees the same codes, the bf16 input and the bias rounded to bf16."""
    import torch
    wl = synth.make_random(24, 96, 256, synth.F16, seed=4, n_outlier_cols=2, bias_sigma=0.01)
    m = make_layer(wl).cuda()
    CB, SCB = m.CB.cpu().numpy(), m.SCB.cpu().numpy()
    m = m.to(torch.bfloat16)
    assert m.SCB.dtype == torch.float32 and np.array_equal(m.SCB.cpu().numpy(), SCB)
    xb = to_torch(wl.X, wl.dtype, "cuda").to(torch.bfloat16)
    y = m(xb)
    torch.cuda.synchronize()
    ref = orc.forward(bits_of(xb), None, synth.BF16, wl.threshold, bias=bits_of(m.bias),
                      weight=(CB, SCB))
    check_y(bits_of(y), ref["Y"], synth.BF16, "forward after .to(bfloat16)")


def test_converted_model_runs_and_keeps_head(orc):
    import torch
    from int8_quantized_matmul_row_amd import nn as n8
    torch.manual_seed(0)
    model = torch.nn.Sequential()
    model.add_module("proj", torch.nn.Linear(256, 128, dtype=torch.float16))
    model.add_module("lm_head", torch.nn.Linear(128, 32, dtype=torch.float16))
    n8.replace_linear_with_8bit(model)
    model = model.cuda()
    x = torch.randn(8, 256, dtype=torch.float16, device="cuda")
    y = model(x)
    torch.cuda.synchronize()
    assert isinstance(model.lm_head, torch.nn.Linear) and y.shape == (8, 32)
    assert torch.isfinite(y.float()).all()


def test_ffn_block_each_projection_matches_oracle(orc):
    """Up -> GeLU -> down with synthetic FFN weights; each projection is checked
    against the oracle on the exact 16-bit input it received."""
    import torch
    from int8_quantized_matmul_row_amd import nn as n8
    d_model, d_ff, M = 512, 1024, 16
    up = synth.make_random(M, d_ff, d_model, synth.F16, seed=11, n_outlier_cols=2,
                           bias_sigma=0.01)
    dn = synth.make_random(M, d_model, d_ff, synth.F16, seed=12, bias_sigma=0.01)
    ffn = n8.FFN8bit.from_weights(to_torch(up.W, synth.F16, "cpu"), to_torch(up.bias, synth.F16, "cpu"),
                                  to_torch(dn.W, synth.F16, "cpu"), to_torch(dn.bias, synth.F16, "cpu"))
    ffn = ffn.cuda()
    x = to_torch(up.X, synth.F16, "cuda")
    h = ffn.up(x)
    g = torch.nn.functional.gelu(h)
    y = ffn.down(g)
    torch.cuda.synchronize()
    dens = ffn.outlier_density()
    log(f"[nn] FFN outlier density {dens}")
    assert dens["up"] == int(ffn.up.last_outlier_count.item()) / d_model
    ref_up = orc.forward(up.X, up.W, synth.F16, 6.0, bias=up.bias)
    check_y(bits_of(h), ref_up["Y"], synth.F16, "FFN up")
    ref_dn = orc.forward(bits_of(g), dn.W, synth.F16, 6.0, bias=dn.bias)
    check_y(bits_of(y), ref_dn["Y"], synth.F16, "FFN down")
    assert torch.equal(ffn(x), y)


def test_checkpoint_of_oracle_codes_matches_oracle(orc, tmp_path):
    """CB and SCB written by the oracle's weight quantization (never quantized
    on the GPU), loaded into a fresh layer: its forward must match the oracle's
    on every stage it exposes ("A Gentle Introduction...", section "Usage":
    the int8 state dict is what is saved and loaded)."""
    import torch
    from int8_quantized_matmul_row_amd import nn as n8
    wl = synth.make_random(40, 192, 320, synth.BF16, seed=21, n_outlier_cols=3, bias_sigma=0.01)
    CB, SCB = orc.quantize_weight(wl.W, wl.dtype)
    host = n8.Linear8bitLt(wl.K, wl.N, dtype=torch.bfloat16)
    host.weight = None
    host.CB, host.SCB = torch.from_numpy(CB), torch.from_numpy(SCB)
    host.bias = torch.nn.Parameter(to_torch(wl.bias, wl.dtype, "cpu"), requires_grad=False)
    path = str(tmp_path / "oracle_codes.safetensors")
    n8.save_quantized(host, path)
    layer = n8.load_quantized(n8.Linear8bitLt(wl.K, wl.N, dtype=torch.float16), path, device="cuda")
    assert layer._dtype == torch.bfloat16 and layer.SCB.dtype == torch.float32
    y = layer(to_torch(wl.X, wl.dtype, "cuda"))
    torch.cuda.synchronize()
    ref = orc.forward(wl.X, None, wl.dtype, wl.threshold, bias=wl.bias, weight=(CB, SCB))
    assert int(layer.last_outlier_count.item()) == len(ref["idx"])
    q = layer._act
    assert np.array_equal(q.CA.cpu().numpy(), ref["CA"])
    assert np.array_equal(q.SCA.cpu().numpy(), ref["SCA"])
    check_y(bits_of(y), ref["Y"], wl.dtype, "layer loaded from oracle codes")


def test_checkpoint_round_trip_gives_identical_output(tmp_path, orc):
    import torch
    from int8_quantized_matmul_row_amd import nn as n8
    wl = synth.make_random(8, 200, 512, synth.BF16, seed=9, n_outlier_cols=2, bias_sigma=0.01)
    m = make_layer(wl).cuda()
    x = to_torch(wl.X, wl.dtype, "cuda")
    y0 = m(x)
    path = str(tmp_path / "q.safetensors")
    n8.save_quantized(m, path)
    fresh = n8.Linear8bitLt(512, 200, dtype=torch.bfloat16)
    n8.load_quantized(fresh, path, device="cuda")
    y1 = fresh(x)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)
    ref = orc.forward(wl.X, wl.W, wl.dtype, wl.threshold, bias=wl.bias)
    assert np.array_equal(fresh.CB.cpu().numpy(), ref["CB"])
    assert np.array_equal(fresh.SCB.cpu().numpy(), ref["SCB"])
    check_y(bits_of(y1), ref["Y"], wl.dtype, "layer loaded from its checkpoint")
