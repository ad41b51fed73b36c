"""Host-side behaviour of the torch-level binding, with the library and torch's
device calls replaced by fakes (no GPU, no kernel):

* every buffer the binding allocates for a call on a given stream is marked as
  used by that stream (record_stream), so that torch's caching allocator cannot
  hand it to other work while that stream's kernels may still use it;
* weights of the wrong type, shape or device, and a bias of the wrong type or
  length, are refused before any pointer reaches the C ABI.
"""
import pytest

import int8_quantized_matmul_row_amd as pkg


class FakeTensor:
    _next = 1 << 20

    def __init__(self, shape, dtype, device="cuda:0"):
        self.shape = tuple(shape)
        self.dtype = dtype
        self.device = device
        self.is_cuda = device.startswith("cuda")
        FakeTensor._next += 1 << 12
        self._ptr = FakeTensor._next
        self.recorded = []

    def data_ptr(self):
        return self._ptr

    def is_contiguous(self):
        return True

    def numel(self):
        n = 1
        for d in self.shape:
            n *= d
        return n

    def record_stream(self, s):
        self.recorded.append(s)

    def zero_(self):
        return self


class FakeStream:
    def __init__(self, handle):
        self.cuda_stream = handle


class FakeTorch:
    float16, bfloat16, float32 = "float16", "bfloat16", "float32"
    int8, uint8, int32 = "int8", "uint8", "int32"

    def __init__(self):
        self.allocated = []
        current = FakeStream(0)
        self.cuda = type("cuda", (), {"current_stream": staticmethod(lambda: current)})

    def empty(self, shape, dtype=None, device=None):
        t = FakeTensor(shape, dtype, str(device))
        self.allocated.append(t)
        return t


class FakeLib:
    def __init__(self):
        self.calls = []

    def __getattr__(self, name):
        if not name.startswith("llmint8_"):
            raise AttributeError(name)

        def fn(*args):
            self.calls.append(name)
            return 4096 if name.endswith("_workspace_size") else 0
        return fn


@pytest.fixture
def fakes(monkeypatch):
    torch, lib = FakeTorch(), FakeLib()
    monkeypatch.setattr(pkg, "_torch", lambda: torch)
    monkeypatch.setattr(pkg, "_lib", lib)
    return torch, lib


def operands(torch, M=64, N=96, K=128, code="int8", scb="float32", bias_dtype="float16", bias_n=None):
    X = FakeTensor((M, K), "float16")
    CB = FakeTensor((N, K), code)
    SCB = FakeTensor((N,), scb)
    bias = FakeTensor((N if bias_n is None else bias_n,), bias_dtype)
    return X, CB, SCB, bias


@pytest.mark.parametrize("variant", ["int8", "fp8"])
def test_buffers_allocated_for_a_stream_are_recorded_on_it(fakes, variant):
    torch, lib = fakes
    X, CB, SCB, bias = operands(torch, code="uint8" if variant == "fp8" else "int8")
    s = FakeStream(1234)
    linear = pkg.linear_fp8 if variant == "fp8" else pkg.linear
    linear(X, CB, SCB, bias=bias, stream=s)
    assert lib.calls[-1] == ("llmint8_linear_fp8" if variant == "fp8" else "llmint8_linear")
    # Y, CA, SCA, idx, n_out, XO and the workspace
    assert len(torch.allocated) == 7
    assert all(t.recorded == [s] for t in torch.allocated)


def test_matmul_and_quantize_act_record_their_buffers(fakes):
    torch, lib = fakes
    X, CB, SCB, bias = operands(torch)
    s = FakeStream(77)
    q = pkg.quantize_act(X, stream=s)
    pkg.matmul(q, CB, SCB, bias=bias, stream=s)
    pkg.quantize_weight(FakeTensor((96, 128), "float16"), stream=s)
    launched = [c for c in lib.calls if not c.endswith("_workspace_size")]
    assert launched == ["llmint8_quantize_act", "llmint8_matmul", "llmint8_quantize_weight"]
    assert torch.allocated and all(t.recorded == [s] for t in torch.allocated)


def test_current_stream_needs_no_record(fakes):
    torch, _ = fakes
    X, CB, SCB, bias = operands(torch)
    pkg.linear(X, CB, SCB, bias=bias)
    assert torch.allocated and not any(t.recorded for t in torch.allocated)


@pytest.mark.parametrize("bad", ["scb_fp16", "cb_shape", "cb_fp8_codes", "cb_on_cpu", "bias_dtype",
                                 "bias_length"])
def test_bad_weights_are_refused_before_the_library(fakes, bad):
    torch, lib = fakes
    kw = {"scb_fp16": dict(scb="float16"), "cb_fp8_codes": dict(code="uint8"),
          "bias_dtype": dict(bias_dtype="bfloat16"), "bias_length": dict(bias_n=95)}.get(bad, {})
    X, CB, SCB, bias = operands(torch, **kw)
    if bad == "cb_shape":
        CB = FakeTensor((96, 64), "int8")
    if bad == "cb_on_cpu":
        CB = FakeTensor((96, 128), "int8", device="cpu")
    with pytest.raises(ValueError):
        pkg.linear(X, CB, SCB, bias=bias)
    assert lib.calls == []
