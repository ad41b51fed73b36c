"""The torch layer over the C ABI (Linear8bitLt), model conversion and the
quantized-weight checkpoint format: host-side behaviour, no GPU needed.

"A Gentle Introduction to 8-bit Matrix Multiplication for transformers at
scale", section "Usage": quantization on placement, the output head kept in
16-bit, CB/SCB held by the layer."""
import numpy as np
import pytest
import torch

from int8_quantized_matmul_row_amd import nn as n8


def test_layer_holds_16bit_weight_until_placed():
    lin = torch.nn.Linear(128, 48, dtype=torch.float16)
    m = n8.Linear8bitLt.from_linear(lin)
    assert not m.quantized and m.CB is None and m.SCB is None
    assert torch.equal(m.weight, lin.weight) and torch.equal(m.bias, lin.bias)
    m = m.to(torch.float16)  # a CPU move does not quantize
    assert not m.quantized


def test_layer_refuses_cpu_forward_and_bad_shapes():
    m = n8.Linear8bitLt.from_linear(torch.nn.Linear(64, 8, dtype=torch.float16))
    with pytest.raises(RuntimeError, match="GPU only"):
        m(torch.zeros(2, 64, dtype=torch.float16))
    with pytest.raises(ValueError, match="multiple of 64"):
        n8.Linear8bitLt(100, 8)
    with pytest.raises(ValueError, match="float16 or bfloat16"):
        n8.Linear8bitLt(64, 8, dtype=torch.float32)


def test_replace_linear_keeps_the_output_head():
    model = torch.nn.Sequential()
    block = torch.nn.Sequential()
    block.add_module("up", torch.nn.Linear(64, 128, dtype=torch.float16))
    block.add_module("act", torch.nn.GELU())
    block.add_module("down", torch.nn.Linear(128, 64, dtype=torch.float16))
    model.add_module("block", block)
    model.add_module("lm_head", torch.nn.Linear(64, 10, dtype=torch.float16))
    n8.replace_linear_with_8bit(model, threshold=5.0, skip=("lm_head", "block.down"))
    assert isinstance(model.block.up, n8.Linear8bitLt) and model.block.up.threshold == 5.0
    assert isinstance(model.block.down, torch.nn.Linear)
    assert isinstance(model.lm_head, torch.nn.Linear)


def test_checkpoint_round_trip_on_host(tmp_path):
    """The file keeps CB (int8), SCB (fp32), bias and the layer settings."""
    rng = np.random.default_rng(5)
    m = n8.Linear8bitLt(128, 16, threshold=4.5)
    m.CB = torch.from_numpy(rng.integers(-127, 128, (16, 128), dtype=np.int8))
    m.SCB = torch.from_numpy(rng.random(16, dtype=np.float32))
    m.bias = torch.nn.Parameter(torch.randn(16).half(), requires_grad=False)
    path = str(tmp_path / "layer.safetensors")
    n8.save_quantized(m, path)
    fresh = n8.Linear8bitLt(128, 16)
    n8.load_quantized(fresh, path, device="cpu")
    assert fresh.weight is None and fresh.threshold == 4.5
    assert torch.equal(fresh.CB, m.CB) and fresh.CB.dtype == torch.int8
    assert torch.equal(fresh.SCB, m.SCB) and fresh.SCB.dtype == torch.float32
    assert torch.equal(fresh.bias, m.bias)
    with pytest.raises(ValueError, match="file has"):
        n8.load_quantized(n8.Linear8bitLt(64, 16), path, device="cpu")


def test_checkpoint_refuses_unquantized_layer(tmp_path):
    m = n8.Linear8bitLt.from_linear(torch.nn.Linear(64, 8, dtype=torch.float16))
    with pytest.raises(RuntimeError, match="not quantized"):
        n8.save_quantized(m, str(tmp_path / "x.safetensors"))


def _quantized_on_host(dtype=torch.float16):
    """A layer holding CB/SCB as if placed (host tensors; no kernel runs)."""
    rng = np.random.default_rng(6)
    m = n8.Linear8bitLt(128, 16, dtype=dtype)
    m.weight = None
    m.CB = torch.from_numpy(rng.integers(-127, 128, (16, 128), dtype=np.int8))
    m.SCB = torch.from_numpy(rng.random(16, dtype=np.float32))
    m.bias = torch.nn.Parameter(torch.randn(16).to(dtype), requires_grad=False)
    return m


@pytest.mark.parametrize("cast", ["half", "bfloat16", "float", "double", "to_f16", "type_f32"])
def test_casts_keep_int8_codes_and_fp32_scales(cast):
    """The recovered weight CB * SCB / 127 ("Usage" section) needs SCB's fp32
    values: no cast may touch them, or CB's int8 codes."""
    m = _quantized_on_host(torch.bfloat16)
    CB, SCB = m.CB.clone(), m.SCB.clone()
    {"half": lambda: m.half(), "bfloat16": lambda: m.bfloat16(), "float": lambda: m.float(),
     "double": lambda: m.double(), "to_f16": lambda: m.to(torch.float16),
     "type_f32": lambda: m.type(torch.float32)}[cast]()
    assert m.CB.dtype == torch.int8 and torch.equal(m.CB, CB)
    assert m.SCB.dtype == torch.float32 and torch.equal(m.SCB, SCB)
    expect = {"half": torch.float16, "to_f16": torch.float16}.get(cast, torch.bfloat16)
    assert m._dtype == expect and m.bias.dtype == expect
