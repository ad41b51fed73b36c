"""Python binding of libllmint8, the LLM.int8() decomposition matmul for MI355X.

Two layers, both argument marshalling only (every step of the computation runs
in the library's HIP kernels):

* ``llmint8_quantize_weight``, ``llmint8_quantize_act``, ``llmint8_matmul``,
  ``llmint8_matmul_profiled`` and the size/status helpers: the C functions of
  ``include/llmint8.h`` with the same names and arguments (device pointers as
  Python ints, ``stream`` as a ``hipStream_t`` int).  They raise
  ``Llmint8Error`` on a non-OK status.
* ``quantize_weight``, ``quantize_act``, ``matmul`` and ``linear``: the same
  calls on torch tensors; torch supplies device memory and the current stream.
* ``*_fp8``: the FP8 (E4M3) variant of the same decomposition (codes as uint8
  tensors; ``t.view(torch.float8_e4m3fn)`` gives their values).

The library must be built (``python -m int8_quantized_matmul_row_amd.build``);
there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import NamedTuple, Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY_PATH = os.path.join(_HERE, "libllmint8.so")

F16 = 0
BF16 = 1
K_ALIGN = 64
K_MAX = 133120
SCRATCH_BYTES = 64 << 20  # LLMINT8_SCRATCH_BYTES: the static scratch of llmint8_linear_noalloc

STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported shape or device", 3: "HIP runtime error"}

EXPORTS = (
    "llmint8_quantize_weight",
    "llmint8_quantize_tensor_workspace_size",
    "llmint8_quantize_tensor",
    "llmint8_quantize_act_workspace_size",
    "llmint8_quantize_act",
    "llmint8_matmul_workspace_size",
    "llmint8_matmul",
    "llmint8_matmul_profiled",
    "llmint8_linear_workspace_size",
    "llmint8_linear",
    "llmint8_linear_profiled",
    "llmint8_linear_noalloc",
    "llmint8_quantize_weight_fp8",
    "llmint8_quantize_act_fp8",
    "llmint8_matmul_fp8",
    "llmint8_matmul_fp8_profiled",
    "llmint8_linear_fp8_workspace_size",
    "llmint8_linear_fp8",
    "llmint8_linear_fp8_profiled",
    "llmint8_peak_mfma",
    "llmint8_status_string",
    "llmint8_last_hip_error",
)


class Llmint8Error(RuntimeError):
    def __init__(self, fn: str, status: int, hip_error: int = 0):
        self.status = status
        self.hip_error = hip_error
        msg = f"{fn}: {STATUS.get(status, 'unknown status')} (status {status}"
        msg += f", hipError {hip_error})" if status == 3 else ")"
        super().__init__(msg)


_lib = None
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_INT = ctypes.c_int


def lib() -> ctypes.CDLL:
    """Load libllmint8.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIBRARY_PATH):
        raise RuntimeError(f"{LIBRARY_PATH} is missing: build it with "
                           "`python -m int8_quantized_matmul_row_amd.build`")
    L = ctypes.CDLL(LIBRARY_PATH)
    L.llmint8_quantize_weight.argtypes = [_P, _INT, _I64, _I64, _P, _P, _P]
    L.llmint8_quantize_tensor_workspace_size.argtypes = [_I64, _I64]
    L.llmint8_quantize_tensor_workspace_size.restype = ctypes.c_size_t
    L.llmint8_quantize_tensor.argtypes = [_P, _INT, _I64, _I64, _P, _P, _P, ctypes.c_size_t, _P]
    L.llmint8_quantize_act_workspace_size.argtypes = [_I64, _I64]
    L.llmint8_quantize_act_workspace_size.restype = ctypes.c_size_t
    L.llmint8_quantize_act.argtypes = [_P, _INT, _I64, _I64, ctypes.c_float, _P, _P, _P, _P, _P,
                                       _P, ctypes.c_size_t, _P]
    L.llmint8_matmul_workspace_size.argtypes = [_I64, _I64, _I64]
    L.llmint8_matmul_workspace_size.restype = ctypes.c_size_t
    mm = [_INT, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
    L.llmint8_matmul.argtypes = mm
    L.llmint8_matmul_profiled.argtypes = mm + [_P, _P]
    L.llmint8_linear_workspace_size.argtypes = [_I64, _I64, _I64]
    L.llmint8_linear_workspace_size.restype = ctypes.c_size_t
    lin = [_P, _INT, _I64, _I64, _I64, ctypes.c_float, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
           ctypes.c_size_t, _P]
    L.llmint8_linear.argtypes = lin
    L.llmint8_linear_profiled.argtypes = lin + [_P, _P]
    L.llmint8_linear_noalloc.argtypes = lin[:-3] + [_P]
    L.llmint8_quantize_weight_fp8.argtypes = L.llmint8_quantize_weight.argtypes
    L.llmint8_quantize_act_fp8.argtypes = L.llmint8_quantize_act.argtypes
    L.llmint8_matmul_fp8.argtypes = mm
    L.llmint8_matmul_fp8_profiled.argtypes = mm + [_P, _P]
    L.llmint8_linear_fp8_workspace_size.argtypes = [_I64, _I64, _I64]
    L.llmint8_linear_fp8_workspace_size.restype = ctypes.c_size_t
    L.llmint8_linear_fp8.argtypes = lin
    L.llmint8_linear_fp8_profiled.argtypes = lin + [_P, _P]
    for f in ("llmint8_quantize_weight", "llmint8_quantize_tensor", "llmint8_quantize_act",
              "llmint8_matmul", "llmint8_matmul_profiled", "llmint8_linear",
              "llmint8_linear_profiled", "llmint8_linear_noalloc", "llmint8_quantize_weight_fp8",
              "llmint8_quantize_act_fp8", "llmint8_matmul_fp8", "llmint8_matmul_fp8_profiled",
              "llmint8_linear_fp8", "llmint8_linear_fp8_profiled"):
        getattr(L, f).restype = _INT
    L.llmint8_peak_mfma.argtypes = [_INT, _P, ctypes.c_size_t, _P, ctypes.c_size_t, _INT, _INT, _P]
    L.llmint8_peak_mfma.restype = _INT
    L.llmint8_status_string.argtypes = [_INT]
    L.llmint8_status_string.restype = ctypes.c_char_p
    L.llmint8_last_hip_error.argtypes = []
    L.llmint8_last_hip_error.restype = _INT
    _lib = L
    return L


def _check(fn: str, status: int):
    if status != 0:
        raise Llmint8Error(fn, status, lib().llmint8_last_hip_error() if status == 3 else 0)


# ---- the C functions, same names and arguments ----------------------------

def llmint8_quantize_weight(W, dtype, N, K, CB, SCB, stream=0):
    _check("llmint8_quantize_weight", lib().llmint8_quantize_weight(W, dtype, N, K, CB, SCB, stream))


def llmint8_quantize_tensor_workspace_size(rows, cols) -> int:
    return int(lib().llmint8_quantize_tensor_workspace_size(rows, cols))


def llmint8_quantize_tensor(A, dtype, rows, cols, Q, scale, workspace, workspace_bytes, stream=0):
    _check("llmint8_quantize_tensor",
           lib().llmint8_quantize_tensor(A, dtype, rows, cols, Q, scale, workspace,
                                         workspace_bytes, stream))


def llmint8_quantize_act_workspace_size(M, K) -> int:
    return int(lib().llmint8_quantize_act_workspace_size(M, K))


def llmint8_quantize_act(X, dtype, M, K, threshold, CA, SCA, outlier_idx, n_outliers, X_outlier,
                         workspace, workspace_bytes, stream=0):
    _check("llmint8_quantize_act",
           lib().llmint8_quantize_act(X, dtype, M, K, ctypes.c_float(threshold), CA, SCA,
                                      outlier_idx, n_outliers, X_outlier, workspace,
                                      workspace_bytes, stream))


def llmint8_matmul_workspace_size(M, N, K) -> int:
    return int(lib().llmint8_matmul_workspace_size(M, N, K))


def llmint8_matmul(dtype, M, N, K, CA, SCA, outlier_idx, n_outliers, X_outlier, CB, SCB, bias,
                   Y, C_i32, workspace, workspace_bytes, stream=0):
    _check("llmint8_matmul",
           lib().llmint8_matmul(dtype, M, N, K, CA, SCA, outlier_idx, n_outliers, X_outlier, CB,
                                SCB, bias, Y, C_i32, workspace, workspace_bytes, stream))


def llmint8_matmul_profiled(dtype, M, N, K, CA, SCA, outlier_idx, n_outliers, X_outlier, CB, SCB,
                            bias, Y, C_i32, workspace, workspace_bytes, stream, start, stop):
    _check("llmint8_matmul_profiled",
           lib().llmint8_matmul_profiled(dtype, M, N, K, CA, SCA, outlier_idx, n_outliers,
                                         X_outlier, CB, SCB, bias, Y, C_i32, workspace,
                                         workspace_bytes, stream, start, stop))


def llmint8_linear_workspace_size(M, N, K) -> int:
    return int(lib().llmint8_linear_workspace_size(M, N, K))


def llmint8_linear(X, dtype, M, N, K, threshold, CB, SCB, bias, Y, CA, SCA, outlier_idx,
                   n_outliers, X_outlier, C_i32, workspace, workspace_bytes, stream=0):
    _check("llmint8_linear",
           lib().llmint8_linear(X, dtype, M, N, K, ctypes.c_float(threshold), CB, SCB, bias, Y, CA,
                                SCA, outlier_idx, n_outliers, X_outlier, C_i32, workspace,
                                workspace_bytes, stream))


def llmint8_linear_profiled(X, dtype, M, N, K, threshold, CB, SCB, bias, Y, CA, SCA, outlier_idx,
                            n_outliers, X_outlier, C_i32, workspace, workspace_bytes, stream,
                            start, stop):
    _check("llmint8_linear_profiled",
           lib().llmint8_linear_profiled(X, dtype, M, N, K, ctypes.c_float(threshold), CB, SCB,
                                         bias, Y, CA, SCA, outlier_idx, n_outliers, X_outlier,
                                         C_i32, workspace, workspace_bytes, stream, start, stop))


def llmint8_linear_noalloc(X, dtype, M, N, K, threshold, CB, SCB, bias, Y, CA, SCA, outlier_idx,
                           n_outliers, X_outlier, C_i32, stream=0):
    _check("llmint8_linear_noalloc",
           lib().llmint8_linear_noalloc(X, dtype, M, N, K, ctypes.c_float(threshold), CB, SCB, bias,
                                        Y, CA, SCA, outlier_idx, n_outliers, X_outlier, C_i32,
                                        stream))


def llmint8_quantize_weight_fp8(W, dtype, N, K, CB, SCB, stream=0):
    _check("llmint8_quantize_weight_fp8",
           lib().llmint8_quantize_weight_fp8(W, dtype, N, K, CB, SCB, stream))


def llmint8_quantize_act_fp8(X, dtype, M, K, threshold, CA, SCA, outlier_idx, n_outliers,
                             X_outlier, workspace, workspace_bytes, stream=0):
    _check("llmint8_quantize_act_fp8",
           lib().llmint8_quantize_act_fp8(X, dtype, M, K, ctypes.c_float(threshold), CA, SCA,
                                          outlier_idx, n_outliers, X_outlier, workspace,
                                          workspace_bytes, stream))


def llmint8_matmul_fp8(dtype, M, N, K, CA, SCA, outlier_idx, n_outliers, X_outlier, CB, SCB,
                       bias, Y, C_f32, workspace, workspace_bytes, stream=0):
    _check("llmint8_matmul_fp8",
           lib().llmint8_matmul_fp8(dtype, M, N, K, CA, SCA, outlier_idx, n_outliers, X_outlier,
                                    CB, SCB, bias, Y, C_f32, workspace, workspace_bytes, stream))


def llmint8_matmul_fp8_profiled(dtype, M, N, K, CA, SCA, outlier_idx, n_outliers, X_outlier, CB,
                                SCB, bias, Y, C_f32, workspace, workspace_bytes, stream, start,
                                stop):
    _check("llmint8_matmul_fp8_profiled",
           lib().llmint8_matmul_fp8_profiled(dtype, M, N, K, CA, SCA, outlier_idx, n_outliers,
                                             X_outlier, CB, SCB, bias, Y, C_f32, workspace,
                                             workspace_bytes, stream, start, stop))


def llmint8_linear_fp8_workspace_size(M, N, K) -> int:
    return int(lib().llmint8_linear_fp8_workspace_size(M, N, K))


def llmint8_linear_fp8(X, dtype, M, N, K, threshold, CB, SCB, bias, Y, CA, SCA, outlier_idx,
                       n_outliers, X_outlier, C_f32, workspace, workspace_bytes, stream=0):
    _check("llmint8_linear_fp8",
           lib().llmint8_linear_fp8(X, dtype, M, N, K, ctypes.c_float(threshold), CB, SCB, bias,
                                    Y, CA, SCA, outlier_idx, n_outliers, X_outlier, C_f32,
                                    workspace, workspace_bytes, stream))


def llmint8_linear_fp8_profiled(X, dtype, M, N, K, threshold, CB, SCB, bias, Y, CA, SCA,
                                outlier_idx, n_outliers, X_outlier, C_f32, workspace,
                                workspace_bytes, stream, start, stop):
    _check("llmint8_linear_fp8_profiled",
           lib().llmint8_linear_fp8_profiled(X, dtype, M, N, K, ctypes.c_float(threshold), CB,
                                             SCB, bias, Y, CA, SCA, outlier_idx, n_outliers,
                                             X_outlier, C_f32, workspace, workspace_bytes,
                                             stream, start, stop))


def llmint8_peak_mfma(fp8, operands, operand_bytes, sink, sink_bytes, blocks, iters, stream=0):
    _check("llmint8_peak_mfma",
           lib().llmint8_peak_mfma(fp8, operands, operand_bytes, sink, sink_bytes, blocks, iters, stream))


def llmint8_status_string(status: int) -> str:
    return lib().llmint8_status_string(status).decode()


def llmint8_last_hip_error() -> int:
    return int(lib().llmint8_last_hip_error())


# ---- torch tensors -----------------------------------------------------------

def _torch():
    import torch
    return torch


def dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float16:
        return F16
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"expected float16 or bfloat16, got {t.dtype}")


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int:
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _empty(shape, dtype, device, stream=None):
    """torch.empty for a buffer the library's kernels use on `stream`.  Given a
    stream, the block is marked as in use by it (record_stream), so that torch's
    caching allocator does not hand it to other work while kernels on that stream
    may still read or write it -- the binding allocates on the current stream, and
    the kernels may run on another."""
    t = _torch().empty(shape, dtype=dtype, device=device)
    if stream is not None:
        t.record_stream(stream)
    return t


def _check_weight(CB, SCB, bias, N, K, device, dtype16, code_dtype):
    """CB [N,K] of code_dtype, SCB [N] float32, bias None or [N] of dtype16, all
    contiguous on `device`: the shapes and types the kernels read."""
    torch = _torch()
    if CB.dtype != code_dtype or tuple(CB.shape) != (N, K):
        raise ValueError(f"CB is {CB.dtype} {tuple(CB.shape)}, expected {code_dtype} ({N}, {K})")
    if SCB.dtype != torch.float32 or tuple(SCB.shape) != (N,):
        raise ValueError(f"SCB is {SCB.dtype} {tuple(SCB.shape)}, expected torch.float32 ({N},)")
    _need(CB, "CB", device)
    _need(SCB, "SCB", device)
    if bias is not None:
        if bias.dtype != dtype16 or bias.numel() != N:
            raise ValueError(f"bias is {bias.dtype} with {bias.numel()} elements, "
                             f"expected {dtype16} with {N}")
        _need(bias, "bias", device)


def _need(t, name, device=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def quantize_weight(W, stream=None, out=None):
    """W [N,K] fp16/bf16 -> (CB int8 [N,K], SCB fp32 [N])."""
    torch = _torch()
    _need(W, "W")
    N, K = W.shape
    CB, SCB = out if out is not None else (
        _empty((N, K), torch.int8, W.device, stream),
        _empty((N,), torch.float32, W.device, stream))
    llmint8_quantize_weight(_ptr(W), dtype_code(W), N, K, _ptr(CB), _ptr(SCB), _stream(stream))
    return CB, SCB


class QuantizedAct(NamedTuple):
    CA: object         # int8 [M,K]
    SCA: object        # fp32 [M]
    idx: object        # int32 [K]; first n_out valid
    n_out: object      # int32 [1] (device)
    XO: object         # 16-bit [M*K]; holds [M, n_pad]
    dtype: int


def alloc_act(M, K, dtype_t, device, fp8: bool = False, stream=None):
    """Output buffers of quantize_act (CA int8) or quantize_act_fp8 (CA uint8)."""
    torch = _torch()
    return QuantizedAct(
        _empty((M, K), torch.uint8 if fp8 else torch.int8, device, stream),
        _empty((M,), torch.float32, device, stream),
        _empty((K,), torch.int32, device, stream),
        _empty((1,), torch.int32, device, stream),
        _empty((max(M * K, 1),), dtype_t, device, stream),
        F16 if dtype_t == torch.float16 else BF16)


def quantize_tensor(A, stream=None):
    """A [R,C] fp16/bf16 -> (Q int8 [R,C], scale fp32 [R]): per-tensor absmax,
    the baseline scheme (one scale for the whole tensor in every row's entry)."""
    torch = _torch()
    _need(A, "A")
    R, C = A.shape
    Q = _empty((R, C), torch.int8, A.device, stream)
    scale = _empty((R,), torch.float32, A.device, stream)
    n = llmint8_quantize_tensor_workspace_size(R, C)
    ws = _empty((max(n, 1),), torch.uint8, A.device, stream)
    llmint8_quantize_tensor(_ptr(A), dtype_code(A), R, C, _ptr(Q), _ptr(scale), _ptr(ws), n,
                            _stream(stream))
    return Q, scale


def matmul_codes(CA, SCA, CB, SCB, dtype_t, bias=None, out=None, stream=None):
    """Y = dequant(CA . CB^T) (+ bias) from int8 codes and row / channel scales
    with no outlier columns -- e.g. two quantize_tensor results (per-tensor
    absmax) -- through llmint8_matmul."""
    M, K = CA.shape
    q = alloc_act(M, K, dtype_t, CA.device, stream=stream)
    q.n_out.zero_()
    q = q._replace(CA=CA, SCA=SCA)
    return matmul(q, CB, SCB, bias=bias, out=out, stream=stream)


def act_workspace(M, K, device, stream=None):
    torch = _torch()
    n = llmint8_quantize_act_workspace_size(M, K)
    return _empty((max(n, 1),), torch.uint8, device, stream), n


def quantize_act(X, threshold: float = 6.0, stream=None, out: Optional[QuantizedAct] = None,
                 workspace=None):
    """X [M,K] fp16/bf16 -> QuantizedAct (outlier columns over all M rows)."""
    _need(X, "X")
    M, K = X.shape
    q = out if out is not None else alloc_act(M, K, X.dtype, X.device, stream=stream)
    ws, nbytes = workspace if workspace is not None else act_workspace(M, K, X.device, stream)
    llmint8_quantize_act(_ptr(X), dtype_code(X), M, K, float(threshold), _ptr(q.CA), _ptr(q.SCA),
                         _ptr(q.idx), _ptr(q.n_out), _ptr(q.XO), _ptr(ws), nbytes,
                         _stream(stream))
    return q


def outlier_columns(q: QuantizedAct):
    """Host copy of the outlier column list (synchronizes)."""
    n = int(q.n_out.item())
    return q.idx[:n].cpu()


def matmul_workspace(M, N, K, device, stream=None):
    """(buffer, bytes) of the optional product workspace (split-K partial
    tiles for shapes with few tiles, and the weight codes at the outlier
    columns, gathered once per call)."""
    torch = _torch()
    n = llmint8_matmul_workspace_size(M, N, K)
    return _empty((max(n, 1),), torch.uint8, device, stream), n


def matmul(q: QuantizedAct, CB, SCB, bias=None, out=None, C_i32=None, stream=None,
           workspace=None, events=None):
    """Y [M,N] = dequant(CA CB^T) + outlier part + bias, in X's dtype.

    workspace: (buffer, bytes); None allocates llmint8_matmul_workspace_size
    bytes, (None, 0) runs without one."""
    torch = _torch()
    M, K = q.CA.shape
    N = CB.shape[0]
    dt_t = torch.float16 if q.dtype == F16 else torch.bfloat16
    _check_weight(CB, SCB, bias, N, K, q.CA.device, dt_t, torch.int8)
    Y = out if out is not None else _empty((M, N), dt_t, q.CA.device, stream)
    if workspace is None:
        workspace = matmul_workspace(M, N, K, q.CA.device, stream)
    ws, nbytes = workspace
    args = (q.dtype, M, N, K, _ptr(q.CA), _ptr(q.SCA), _ptr(q.idx), _ptr(q.n_out), _ptr(q.XO),
            _ptr(CB), _ptr(SCB), _ptr(bias), _ptr(Y), _ptr(C_i32), _ptr(ws), nbytes,
            _stream(stream))
    if events is None:
        llmint8_matmul(*args)
    else:
        llmint8_matmul_profiled(*args, events[0], events[1])
    return Y


def linear_workspace(M, N, K, device, stream=None):
    torch = _torch()
    n = llmint8_linear_workspace_size(M, N, K)
    return _empty((max(n, 1),), torch.uint8, device, stream), n


def linear(X, CB, SCB, bias=None, threshold: float = 6.0, stream=None, out=None,
           act: Optional[QuantizedAct] = None, C_i32=None, workspace=None, events=None):
    """Y = X . W^T through LLM.int8() in one call, W given as (CB, SCB).

    Returns (Y, QuantizedAct): the activation outputs are filled as by
    quantize_act."""
    torch = _torch()
    _need(X, "X")
    M, K = X.shape
    N = CB.shape[0]
    _check_weight(CB, SCB, bias, N, K, X.device, X.dtype, torch.int8)
    q = act if act is not None else alloc_act(M, K, X.dtype, X.device, stream=stream)
    Y = out if out is not None else _empty((M, N), X.dtype, X.device, stream)
    if workspace is None:
        workspace = linear_workspace(M, N, K, X.device, stream)
    ws, nbytes = workspace
    args = (_ptr(X), dtype_code(X), M, N, K, float(threshold), _ptr(CB), _ptr(SCB), _ptr(bias),
            _ptr(Y), _ptr(q.CA), _ptr(q.SCA), _ptr(q.idx), _ptr(q.n_out), _ptr(q.XO), _ptr(C_i32),
            _ptr(ws), nbytes, _stream(stream))
    if events is None:
        llmint8_linear(*args)
    else:
        llmint8_linear_profiled(*args, events[0], events[1])
    return Y, q


# ---- FP8 (E4M3) variant --------------------------------------------------------

def quantize_weight_fp8(W, stream=None, out=None):
    """W [N,K] fp16/bf16 -> (CB uint8 E4M3 codes [N,K], SCB fp32 [N])."""
    torch = _torch()
    _need(W, "W")
    N, K = W.shape
    CB, SCB = out if out is not None else (
        _empty((N, K), torch.uint8, W.device, stream),
        _empty((N,), torch.float32, W.device, stream))
    llmint8_quantize_weight_fp8(_ptr(W), dtype_code(W), N, K, _ptr(CB), _ptr(SCB),
                                _stream(stream))
    return CB, SCB


def quantize_act_fp8(X, threshold: float = 6.0, stream=None, out: Optional[QuantizedAct] = None,
                     workspace=None):
    """X [M,K] fp16/bf16 -> QuantizedAct with CA as uint8 E4M3 codes."""
    _need(X, "X")
    M, K = X.shape
    q = out if out is not None else alloc_act(M, K, X.dtype, X.device, fp8=True,
                                                  stream=stream)
    ws, nbytes = workspace if workspace is not None else act_workspace(M, K, X.device, stream)
    llmint8_quantize_act_fp8(_ptr(X), dtype_code(X), M, K, float(threshold), _ptr(q.CA),
                             _ptr(q.SCA), _ptr(q.idx), _ptr(q.n_out), _ptr(q.XO), _ptr(ws),
                             nbytes, _stream(stream))
    return q


def matmul_fp8(q: QuantizedAct, CB, SCB, bias=None, out=None, C_f32=None, stream=None,
               workspace=None, events=None):
    """The FP8 product Y [M,N] from quantize_act_fp8 / quantize_weight_fp8 outputs
    (workspace as in matmul)."""
    torch = _torch()
    M, K = q.CA.shape
    N = CB.shape[0]
    dt_t = torch.float16 if q.dtype == F16 else torch.bfloat16
    _check_weight(CB, SCB, bias, N, K, q.CA.device, dt_t, torch.uint8)
    Y = out if out is not None else _empty((M, N), dt_t, q.CA.device, stream)
    if workspace is None:
        workspace = matmul_workspace(M, N, K, q.CA.device, stream)
    ws, nbytes = workspace
    args = (q.dtype, M, N, K, _ptr(q.CA), _ptr(q.SCA), _ptr(q.idx), _ptr(q.n_out), _ptr(q.XO),
            _ptr(CB), _ptr(SCB), _ptr(bias), _ptr(Y), _ptr(C_f32), _ptr(ws), nbytes,
            _stream(stream))
    if events is None:
        llmint8_matmul_fp8(*args)
    else:
        llmint8_matmul_fp8_profiled(*args, events[0], events[1])
    return Y


def linear_fp8_workspace(M, N, K, device, stream=None):
    torch = _torch()
    n = llmint8_linear_fp8_workspace_size(M, N, K)
    return _empty((max(n, 1),), torch.uint8, device, stream), n


def linear_fp8(X, CB, SCB, bias=None, threshold: float = 6.0, stream=None, out=None,
               act: Optional[QuantizedAct] = None, C_f32=None, workspace=None, events=None):
    """Y = X . W^T through the FP8 variant in one call, W given as (CB, SCB) from
    quantize_weight_fp8.  Returns (Y, QuantizedAct)."""
    torch = _torch()
    _need(X, "X")
    M, K = X.shape
    N = CB.shape[0]
    _check_weight(CB, SCB, bias, N, K, X.device, X.dtype, torch.uint8)
    q = act if act is not None else alloc_act(M, K, X.dtype, X.device, fp8=True, stream=stream)
    Y = out if out is not None else _empty((M, N), X.dtype, X.device, stream)
    if workspace is None:
        workspace = linear_fp8_workspace(M, N, K, X.device, stream)
    ws, nbytes = workspace
    args = (_ptr(X), dtype_code(X), M, N, K, float(threshold), _ptr(CB), _ptr(SCB), _ptr(bias),
            _ptr(Y), _ptr(q.CA), _ptr(q.SCA), _ptr(q.idx), _ptr(q.n_out), _ptr(q.XO), _ptr(C_f32),
            _ptr(ws), nbytes, _stream(stream))
    if events is None:
        llmint8_linear_fp8(*args)
    else:
        llmint8_linear_fp8_profiled(*args, events[0], events[1])
    return Y, q
