"""torch modules over the C ABI: an LLM.int8() linear layer, model conversion,
a chained FFN block, and quantized-weight checkpoints.

"A Gentle Introduction to 8-bit Matrix Multiplication for transformers at
scale", section "Usage": the layer is built from 16-bit weights, is quantized
once when it is placed on the GPU (its int8 weight and per-output-channel
scales become `CB` and `SCB`), takes 16-bit activations and returns 16-bit
outputs, with outlier columns at threshold 6.0; the model's output head stays
in 16-bit.  The same page (and "Hugging Face 将 LLM.int8() 8 位矩阵乘法集成到
Transformers 和 Accelerate 中") notes that saving the int8 weights was not yet
possible; `save_quantized` / `load_quantized` store CB and SCB so that weight
quantization can run offline.

Every step of the forward runs in libllmint8's kernels; torch only holds the
device buffers.  There is no CPU forward: calling the layer on a CPU tensor
raises.
"""
from __future__ import annotations

import json
from typing import Iterable, Optional

import torch

from . import QuantizedAct, alloc_act, linear, linear_workspace, quantize_weight

__all__ = ["Linear8bitLt", "replace_linear_with_8bit", "FFN8bit", "save_quantized",
           "load_quantized"]


class Linear8bitLt(torch.nn.Module):
    """y = x W^T + b through the LLM.int8() decomposition.

    The 16-bit `weight` is kept until the module is moved to a GPU; the move
    quantizes it once into the buffers `CB` [out, in] int8 and `SCB` [out]
    fp32 and, unless `has_fp16_weights`, drops the 16-bit copy.  Moving or
    copying the module again never quantizes twice.  (A module created on the
    GPU holds an uninitialized weight: fill it, then call .cuda() to quantize.)
    in_features must be a multiple of 64.

    Casts: CB stays int8 and SCB float32 under any cast (.half(), .to(dtype),
    .type(...)); they only change device.  A cast between float16 and bfloat16
    switches the layer's 16-bit type (its input, output and bias); a cast to
    any other floating type leaves the 16-bit type as it is.
    """

    def __init__(self, in_features: int, out_features: int, bias: bool = True,
                 has_fp16_weights: bool = False, threshold: float = 6.0,
                 dtype: torch.dtype = torch.float16, device=None):
        super().__init__()
        if in_features % 64 != 0:
            raise ValueError(f"in_features must be a multiple of 64, got {in_features}")
        if dtype not in (torch.float16, torch.bfloat16):
            raise ValueError(f"dtype must be float16 or bfloat16, got {dtype}")
        self.in_features, self.out_features = in_features, out_features
        self.threshold = float(threshold)
        self.has_fp16_weights = has_fp16_weights
        self.weight = torch.nn.Parameter(
            torch.empty((out_features, in_features), dtype=dtype, device=device),
            requires_grad=False)
        self.bias = (torch.nn.Parameter(torch.zeros(out_features, dtype=dtype, device=device),
                                        requires_grad=False) if bias else None)
        self.register_buffer("CB", None)
        self.register_buffer("SCB", None)
        self._dtype = dtype
        self._act: Optional[QuantizedAct] = None
        self._ws = None
        self.last_outlier_count: Optional[torch.Tensor] = None  # device int32, no sync

    @property
    def quantized(self) -> bool:
        return self.CB is not None

    def _quantize(self):
        if self.quantized or self.weight is None or not self.weight.is_cuda:
            return
        CB, SCB = quantize_weight(self.weight.data)
        self.CB, self.SCB = CB, SCB
        if not self.has_fp16_weights:
            self.weight = None

    def _apply(self, fn, *args, **kwargs):
        # CB (int8) and SCB (fp32 scales) keep their dtypes whatever the cast:
        # they move by device only.  The layer's 16-bit type (input, output,
        # bias, any kept 16-bit weight) follows a cast between float16 and
        # bfloat16; a cast to another floating type moves the layer's tensors
        # but keeps their 16-bit type, since the kernels take 16-bit data only.
        here = self.SCB.device if self.quantized else (
            self.weight.device if self.weight is not None else torch.device("cpu"))
        probe = fn(torch.zeros(1, dtype=self._dtype, device=here))
        target = probe.device
        new16 = probe.dtype if probe.dtype in (torch.float16, torch.bfloat16) else self._dtype
        CB, SCB = self.CB, self.SCB
        self.CB = self.SCB = None

        def move(t):
            return t.to(device=target, dtype=new16 if t.is_floating_point() else None)

        try:
            super()._apply(move, *args, **kwargs)
        finally:
            if CB is not None:
                self.CB, self.SCB = CB.to(target), SCB.to(target)
        if new16 != self._dtype:
            self._dtype = new16
            self._act, self._ws = None, None
        self._quantize()
        return self

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        if not self.quantized:
            raise RuntimeError("Linear8bitLt runs on the GPU only: move it with .cuda() / "
                               ".to('cuda') first (that quantizes the weight)")
        if x.dtype != self._dtype:
            raise ValueError(f"input dtype {x.dtype} does not match the layer's {self._dtype}")
        if x.shape[-1] != self.in_features:
            raise ValueError(f"input has {x.shape[-1]} features, expected {self.in_features}")
        lead = x.shape[:-1]
        X = x.reshape(-1, self.in_features)
        if not X.is_contiguous():
            X = X.contiguous()
        M = X.shape[0]
        if (self._act is None or self._act.CA.shape[0] != M or self._act.CA.device != X.device
                or self._act.XO.dtype != X.dtype):
            self._act = alloc_act(M, self.in_features, X.dtype, X.device)
            self._ws = linear_workspace(M, self.out_features, self.in_features, X.device)
        Y, q = linear(X, self.CB, self.SCB, bias=self.bias, threshold=self.threshold,
                      act=self._act, workspace=self._ws)
        self.last_outlier_count = q.n_out
        return Y.reshape(*lead, self.out_features)

    @classmethod
    def from_linear(cls, lin: torch.nn.Linear, threshold: float = 6.0,
                    has_fp16_weights: bool = False) -> "Linear8bitLt":
        """A Linear8bitLt holding lin's weight and bias (quantized when, or if,
        lin's weight already is, on the GPU)."""
        dtype = lin.weight.dtype
        m = cls(lin.in_features, lin.out_features, bias=lin.bias is not None,
                has_fp16_weights=has_fp16_weights, threshold=threshold, dtype=dtype)
        m.weight = torch.nn.Parameter(lin.weight.data.detach().clone(), requires_grad=False)
        if lin.bias is not None:
            m.bias = torch.nn.Parameter(lin.bias.data.detach().clone(), requires_grad=False)
        m._quantize()
        return m

    def extra_repr(self) -> str:
        return (f"in_features={self.in_features}, out_features={self.out_features}, "
                f"bias={self.bias is not None}, threshold={self.threshold}, "
                f"quantized={self.quantized}")


def replace_linear_with_8bit(model: torch.nn.Module, threshold: float = 6.0,
                             skip: Iterable[str] = ("lm_head",)) -> torch.nn.Module:
    """Replace every torch.nn.Linear of `model` (in place) by a Linear8bitLt,
    except modules whose name (or dotted path) is in `skip` -- by default the
    output head, which the pages keep in 16-bit."""
    skip = set(skip)
    for name, child in list(model.named_children()):
        if name in skip:
            continue
        if isinstance(child, torch.nn.Linear):
            setattr(model, name, Linear8bitLt.from_linear(child, threshold=threshold))
        else:
            sub_skip = {s.split(".", 1)[1] for s in skip if s.startswith(name + ".")}
            replace_linear_with_8bit(child, threshold, skip=(skip - {name}) | sub_skip)
    return model


class FFN8bit(torch.nn.Module):
    """A transformer feed-forward block, up-projection -> GeLU -> down-projection,
    with both projections in LLM.int8().  `outlier_density()` reports, after a
    forward, the fraction of feature columns each projection treated as
    outliers (read from the device counts)."""

    def __init__(self, up: Linear8bitLt, down: Linear8bitLt):
        super().__init__()
        if up.out_features != down.in_features:
            raise ValueError("up.out_features must equal down.in_features")
        self.up, self.down = up, down

    @classmethod
    def from_weights(cls, W_up, b_up, W_down, b_down, threshold: float = 6.0) -> "FFN8bit":
        """W_up [d_ff, d_model], W_down [d_model, d_ff] (16-bit, any device)."""
        def layer(W, b):
            lin = torch.nn.Linear(W.shape[1], W.shape[0], bias=b is not None, dtype=W.dtype,
                                  device=W.device)
            with torch.no_grad():
                lin.weight.copy_(W)
                if b is not None:
                    lin.bias.copy_(b)
            return Linear8bitLt.from_linear(lin, threshold=threshold)
        return cls(layer(W_up, b_up), layer(W_down, b_down))

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        return self.down(torch.nn.functional.gelu(self.up(x)))

    def outlier_density(self) -> dict:
        out = {}
        for name, layer in (("up", self.up), ("down", self.down)):
            n = layer.last_outlier_count
            out[name] = None if n is None else int(n.item()) / layer.in_features
        return out


def save_quantized(module: torch.nn.Module, path: str) -> None:
    """Write every quantized Linear8bitLt of `module` (CB, SCB, bias) to a
    safetensors file, with the layer settings in its metadata."""
    from safetensors.torch import save_file
    tensors, meta = {}, {}
    for name, m in module.named_modules():
        if isinstance(m, Linear8bitLt):
            if not m.quantized:
                raise RuntimeError(f"layer '{name}' is not quantized yet (move it to the GPU)")
            key = name or "_"
            tensors[f"{key}.CB"] = m.CB.detach().cpu().contiguous()
            tensors[f"{key}.SCB"] = m.SCB.detach().cpu().contiguous()
            if m.bias is not None:
                tensors[f"{key}.bias"] = m.bias.detach().cpu().contiguous()
            meta[key] = {"in_features": m.in_features, "out_features": m.out_features,
                         "threshold": m.threshold, "dtype": str(m._dtype).replace("torch.", ""),
                         "bias": m.bias is not None}
    save_file(tensors, path, metadata={"llmint8_layers": json.dumps(meta)})


def load_quantized(module: torch.nn.Module, path: str, device="cuda") -> torch.nn.Module:
    """Fill the Linear8bitLt layers of `module` from a file written by
    save_quantized: CB and SCB are loaded as they are (no weight quantization
    runs) and placed on `device`."""
    from safetensors import safe_open
    with safe_open(path, framework="pt") as f:
        meta = json.loads(f.metadata()["llmint8_layers"])
        for name, m in module.named_modules():
            if not isinstance(m, Linear8bitLt):
                continue
            key = name or "_"
            if key not in meta:
                raise KeyError(f"layer '{name}' is not in {path}")
            info = meta[key]
            if (info["in_features"], info["out_features"]) != (m.in_features, m.out_features):
                raise ValueError(f"layer '{name}': file has {info['out_features']}x"
                                 f"{info['in_features']}, module {m.out_features}x{m.in_features}")
            CB, SCB = f.get_tensor(f"{key}.CB"), f.get_tensor(f"{key}.SCB")
            N, K = m.out_features, m.in_features
            if CB.dtype != torch.int8 or tuple(CB.shape) != (N, K):
                raise ValueError(f"layer '{name}': CB is {CB.dtype} {tuple(CB.shape)}, "
                                 f"expected torch.int8 ({N}, {K})")
            if SCB.dtype != torch.float32 or tuple(SCB.shape) != (N,):
                raise ValueError(f"layer '{name}': SCB is {SCB.dtype} {tuple(SCB.shape)}, "
                                 f"expected torch.float32 ({N},)")
            dtype = getattr(torch, info["dtype"])
            m.weight = None
            m.CB, m.SCB = CB.to(device), SCB.to(device)
            m.threshold = float(info["threshold"])
            m._dtype = dtype
            m._act, m._ws = None, None
            if info["bias"]:
                m.bias = torch.nn.Parameter(f.get_tensor(f"{key}.bias").to(device, dtype),
                                            requires_grad=False)
            else:
                m.bias = None
    return module
