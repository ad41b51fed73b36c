"""ctypes wrapper of the CPU oracle (llmint8_oracle.c).

TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this package.  The product path (the HIP library
and its Python binding) never imports it.

Arrays are numpy; 16-bit tensors travel as uint16 bit patterns plus a dtype
code (0 = fp16, 1 = bf16).  FP8 (E4M3) codes travel as uint8.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "llmint8_oracle.c")
LIBRARY = os.path.join(_HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
          "-Wall", "-Wextra"]


def build(out_path: str = LIBRARY, source: str = SOURCE, extra_flags=()) -> str:
    """Compile the oracle (or another copy of its source) with gcc."""
    cmd = ["gcc", *CFLAGS, *extra_flags, source, "-o", out_path, "-lm"]
    tmp = out_path + ".tmp"
    cmd[cmd.index(out_path)] = tmp
    subprocess.run(cmd, check=True)
    os.replace(tmp, out_path)
    return out_path


class OracleError(RuntimeError):
    pass


_P = ctypes.c_void_p
_I64 = ctypes.c_int64


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


class Oracle:
    """The oracle's functions on numpy arrays."""

    def __init__(self, path: str = LIBRARY):
        if not os.path.exists(path):
            build(path)
        self.path = path
        lib = ctypes.CDLL(path)
        lib.oracle_widen.argtypes = [_P, ctypes.c_int, _I64, _P]
        lib.oracle_quantize_weight.argtypes = [_P, ctypes.c_int, _I64, _I64, _P, _P]
        lib.oracle_quantize_tensor.argtypes = [_P, ctypes.c_int, _I64, _I64, _P, _P]
        lib.oracle_quantize_act.argtypes = [_P, ctypes.c_int, _I64, _I64, ctypes.c_float,
                                            _P, _P, _P, _P, _P]
        lib.oracle_int8_rows.argtypes = [_P, _P, _I64, _I64, _I64, _P, _I64, _P]
        lib.oracle_recover_weight.argtypes = [_P, _P, _I64, _I64, _P]
        lib.oracle_output_rows.argtypes = [_P, _P, _P, _P, ctypes.c_int, _P, ctypes.c_int32,
                                           _P, _P, _I64, _I64, _I64, _P, _I64, _P]
        lib.oracle_e4m3_encode.argtypes = [_P, _I64, _P]
        lib.oracle_e4m3_decode.argtypes = [_P, _I64, _P]
        lib.oracle_quantize_weight_fp8.argtypes = [_P, ctypes.c_int, _I64, _I64, _P, _P]
        lib.oracle_quantize_act_fp8.argtypes = [_P, ctypes.c_int, _I64, _I64, ctypes.c_float,
                                                _P, _P, _P, _P, _P]
        lib.oracle_fp8_rows.argtypes = [_P, _P, _I64, _I64, _I64, _P, _I64, _P]
        lib.oracle_output_rows_fp8.argtypes = [_P, _P, _P, _P, ctypes.c_int, _P, ctypes.c_int32,
                                               _P, _P, _I64, _I64, _I64, _P, _I64, _P]
        for f in ("oracle_widen", "oracle_quantize_weight", "oracle_quantize_tensor",
                  "oracle_quantize_act",
                  "oracle_int8_rows", "oracle_recover_weight", "oracle_output_rows",
                  "oracle_e4m3_encode", "oracle_e4m3_decode", "oracle_quantize_weight_fp8",
                  "oracle_quantize_act_fp8", "oracle_fp8_rows", "oracle_output_rows_fp8"):
            getattr(lib, f).restype = ctypes.c_int
        self.lib = lib

    @staticmethod
    def _check(rc: int, what: str):
        if rc != 0:
            raise OracleError(f"{what} failed with code {rc}")

    def widen(self, bits: np.ndarray, dtype: int) -> np.ndarray:
        bits = np.ascontiguousarray(bits, dtype=np.uint16)
        out = np.empty(bits.shape, dtype=np.float32)
        self._check(self.lib.oracle_widen(_ptr(bits), dtype, bits.size, _ptr(out)), "widen")
        return out

    def quantize_weight(self, W: np.ndarray, dtype: int):
        """W uint16 [N,K] -> (CB int8 [N,K], SCB float32 [N])."""
        W = np.ascontiguousarray(W, dtype=np.uint16)
        N, K = W.shape
        CB = np.empty((N, K), dtype=np.int8)
        SCB = np.empty(N, dtype=np.float32)
        self._check(self.lib.oracle_quantize_weight(_ptr(W), dtype, N, K, _ptr(CB), _ptr(SCB)),
                    "quantize_weight")
        return CB, SCB

    def quantize_tensor(self, A: np.ndarray, dtype: int):
        """A uint16 [R,C] -> (Q int8 [R,C], scale float32 [R]): one absmax for the
        whole tensor, written to every row's scale."""
        A = np.ascontiguousarray(A, dtype=np.uint16)
        R, C = A.shape
        Q = np.empty((R, C), dtype=np.int8)
        scale = np.empty(R, dtype=np.float32)
        self._check(self.lib.oracle_quantize_tensor(_ptr(A), dtype, R, C, _ptr(Q), _ptr(scale)),
                    "quantize_tensor")
        return Q, scale

    def quantize_act(self, X: np.ndarray, dtype: int, threshold: float):
        """X uint16 [M,K] -> (CA int8 [M,K], SCA f32 [M], idx int32 [n_out], XO uint16 [M,n_out])."""
        X = np.ascontiguousarray(X, dtype=np.uint16)
        M, K = X.shape
        CA = np.empty((M, K), dtype=np.int8)
        SCA = np.empty(M, dtype=np.float32)
        idx = np.empty(max(K, 1), dtype=np.int32)
        n_out = np.zeros(1, dtype=np.int32)
        XO = np.empty(max(M * K, 1), dtype=np.uint16)
        self._check(self.lib.oracle_quantize_act(_ptr(X), dtype, M, K, ctypes.c_float(threshold),
                                                 _ptr(CA), _ptr(SCA), _ptr(idx), _ptr(n_out),
                                                 _ptr(XO)), "quantize_act")
        n = int(n_out[0])
        return CA, SCA, idx[:n].copy(), XO[:M * n].reshape(M, n).copy()

    def int8_rows(self, CA: np.ndarray, CB: np.ndarray, rows=None) -> np.ndarray:
        """int32 C [len(rows), N] = CA[rows] . CB^T (exact)."""
        CA = np.ascontiguousarray(CA, dtype=np.int8)
        CB = np.ascontiguousarray(CB, dtype=np.int8)
        M, K = CA.shape
        N = CB.shape[0]
        assert CB.shape[1] == K
        rows = np.arange(M, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
        C = np.empty((len(rows), N), dtype=np.int32)
        self._check(self.lib.oracle_int8_rows(_ptr(CA), _ptr(CB), M, N, K, _ptr(rows), len(rows),
                                              _ptr(C)), "int8_rows")
        return C

    def recover_weight(self, CB: np.ndarray, SCB: np.ndarray) -> np.ndarray:
        CB = np.ascontiguousarray(CB, dtype=np.int8)
        SCB = np.ascontiguousarray(SCB, dtype=np.float32)
        N, K = CB.shape
        out = np.empty((N, K), dtype=np.float64)
        self._check(self.lib.oracle_recover_weight(_ptr(CB), _ptr(SCB), N, K, _ptr(out)),
                    "recover_weight")
        return out

    def output_rows(self, C, SCA, SCB, X, dtype, idx, CB, bias, rows=None) -> np.ndarray:
        """float64 Y [len(rows), N]; C holds the int8 product of the same rows."""
        X = np.ascontiguousarray(X, dtype=np.uint16)
        M, K = X.shape
        CB = np.ascontiguousarray(CB, dtype=np.int8)
        N = CB.shape[0]
        rows = np.arange(M, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
        C = np.ascontiguousarray(C, dtype=np.int32)
        assert C.shape == (len(rows), N)
        SCA = np.ascontiguousarray(SCA, dtype=np.float32)
        SCB = np.ascontiguousarray(SCB, dtype=np.float32)
        idx = np.ascontiguousarray(idx, dtype=np.int32)
        bias = None if bias is None else np.ascontiguousarray(bias, dtype=np.uint16)
        Y = np.empty((len(rows), N), dtype=np.float64)
        self._check(self.lib.oracle_output_rows(_ptr(C), _ptr(SCA), _ptr(SCB), _ptr(X), dtype,
                                                _ptr(idx), ctypes.c_int32(len(idx)), _ptr(CB),
                                                _ptr(bias), M, N, K, _ptr(rows), len(rows),
                                                _ptr(Y)), "output_rows")
        return Y

    # -- FP8 (E4M3) variant -------------------------------------------------------
    def e4m3_encode(self, x: np.ndarray) -> np.ndarray:
        """float32 values -> uint8 E4M3 codes (nearest, ties to even)."""
        x = np.ascontiguousarray(x, dtype=np.float32)
        out = np.empty(x.shape, dtype=np.uint8)
        self._check(self.lib.oracle_e4m3_encode(_ptr(x), x.size, _ptr(out)), "e4m3_encode")
        return out

    def e4m3_decode(self, c: np.ndarray) -> np.ndarray:
        """uint8 E4M3 codes -> float64 values (NaN for S.1111.111)."""
        c = np.ascontiguousarray(c, dtype=np.uint8)
        out = np.empty(c.shape, dtype=np.float64)
        self._check(self.lib.oracle_e4m3_decode(_ptr(c), c.size, _ptr(out)), "e4m3_decode")
        return out

    def quantize_weight_fp8(self, W: np.ndarray, dtype: int):
        """W uint16 [N,K] -> (CB uint8 E4M3 [N,K], SCB float32 [N])."""
        W = np.ascontiguousarray(W, dtype=np.uint16)
        N, K = W.shape
        CB = np.empty((N, K), dtype=np.uint8)
        SCB = np.empty(N, dtype=np.float32)
        self._check(self.lib.oracle_quantize_weight_fp8(_ptr(W), dtype, N, K, _ptr(CB), _ptr(SCB)),
                    "quantize_weight_fp8")
        return CB, SCB

    def quantize_act_fp8(self, X: np.ndarray, dtype: int, threshold: float):
        """X uint16 [M,K] -> (CA uint8 E4M3 [M,K], SCA f32 [M], idx int32 [n_out],
        XO uint16 [M,n_out])."""
        X = np.ascontiguousarray(X, dtype=np.uint16)
        M, K = X.shape
        CA = np.empty((M, K), dtype=np.uint8)
        SCA = np.empty(M, dtype=np.float32)
        idx = np.empty(max(K, 1), dtype=np.int32)
        n_out = np.zeros(1, dtype=np.int32)
        XO = np.empty(max(M * K, 1), dtype=np.uint16)
        self._check(self.lib.oracle_quantize_act_fp8(_ptr(X), dtype, M, K, ctypes.c_float(threshold),
                                                     _ptr(CA), _ptr(SCA), _ptr(idx), _ptr(n_out),
                                                     _ptr(XO)), "quantize_act_fp8")
        n = int(n_out[0])
        return CA, SCA, idx[:n].copy(), XO[:M * n].reshape(M, n).copy()

    def fp8_rows(self, CA: np.ndarray, CB: np.ndarray, rows=None) -> np.ndarray:
        """float64 C [len(rows), N] = value(CA[rows]) . value(CB)^T (exact)."""
        CA = np.ascontiguousarray(CA, dtype=np.uint8)
        CB = np.ascontiguousarray(CB, dtype=np.uint8)
        M, K = CA.shape
        N = CB.shape[0]
        assert CB.shape[1] == K
        rows = np.arange(M, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
        C = np.empty((len(rows), N), dtype=np.float64)
        self._check(self.lib.oracle_fp8_rows(_ptr(CA), _ptr(CB), M, N, K, _ptr(rows), len(rows),
                                             _ptr(C)), "fp8_rows")
        return C

    def output_rows_fp8(self, C, SCA, SCB, X, dtype, idx, CB, bias, rows=None) -> np.ndarray:
        """float64 Y [len(rows), N]; C holds the FP8 product of the same rows."""
        X = np.ascontiguousarray(X, dtype=np.uint16)
        M, K = X.shape
        CB = np.ascontiguousarray(CB, dtype=np.uint8)
        N = CB.shape[0]
        rows = np.arange(M, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
        C = np.ascontiguousarray(C, dtype=np.float64)
        assert C.shape == (len(rows), N)
        SCA = np.ascontiguousarray(SCA, dtype=np.float32)
        SCB = np.ascontiguousarray(SCB, dtype=np.float32)
        idx = np.ascontiguousarray(idx, dtype=np.int32)
        bias = None if bias is None else np.ascontiguousarray(bias, dtype=np.uint16)
        Y = np.empty((len(rows), N), dtype=np.float64)
        self._check(self.lib.oracle_output_rows_fp8(_ptr(C), _ptr(SCA), _ptr(SCB), _ptr(X), dtype,
                                                    _ptr(idx), ctypes.c_int32(len(idx)), _ptr(CB),
                                                    _ptr(bias), M, N, K, _ptr(rows), len(rows),
                                                    _ptr(Y)), "output_rows_fp8")
        return Y

    def forward_fp8(self, X, W, dtype, threshold, bias=None, rows=None, weight=None):
        """All stages of the FP8 variant for the given rows (default: all)."""
        CB, SCB = weight if weight is not None else self.quantize_weight_fp8(W, dtype)
        CA, SCA, idx, XO = self.quantize_act_fp8(X, dtype, threshold)
        C = self.fp8_rows(CA, CB, rows)
        Y = self.output_rows_fp8(C, SCA, SCB, X, dtype, idx, CB, bias, rows)
        return dict(CB=CB, SCB=SCB, CA=CA, SCA=SCA, idx=idx, XO=XO, C=C, Y=Y)

    # -- whole forward ---------------------------------------------------------
    def forward(self, X, W, dtype, threshold, bias=None, rows=None, weight=None):
        """All stages for the given rows (default: all).  Returns a dict."""
        CB, SCB = weight if weight is not None else self.quantize_weight(W, dtype)
        CA, SCA, idx, XO = self.quantize_act(X, dtype, threshold)
        C = self.int8_rows(CA, CB, rows)
        Y = self.output_rows(C, SCA, SCB, X, dtype, idx, CB, bias, rows)
        return dict(CB=CB, SCB=SCB, CA=CA, SCA=SCA, idx=idx, XO=XO, C=C, Y=Y)


def forward_rows_threaded(orc: Oracle, act, weight, X, dtype, bias, rows, threads: int,
                          fp8: bool = False):
    """C and Y of `rows` from the activation outputs act = (CA, SCA, idx, XO) and
    weight = (CB, SCB): the unchanged per-row functions (int8_rows or fp8_rows, then
    output_rows or output_rows_fp8), each thread on a contiguous chunk of the rows.
    Once the outlier set and the scales are fixed the rows are independent, so the
    result is the same for every thread count.  ctypes releases the GIL for the
    duration of each foreign call, so the chunks run on separate cores."""
    import concurrent.futures as cf
    CA, SCA, idx, _ = act
    CB, SCB = weight
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    threads = max(1, min(int(threads), len(rows)))
    chunks = np.array_split(rows, threads)
    prod = orc.fp8_rows if fp8 else orc.int8_rows
    out = orc.output_rows_fp8 if fp8 else orc.output_rows

    def one(r):
        C = prod(CA, CB, r)
        return C, out(C, SCA, SCB, X, dtype, idx, CB, bias, r)

    if threads == 1:
        parts = [one(rows)]
    else:
        with cf.ThreadPoolExecutor(max_workers=threads) as ex:
            parts = list(ex.map(one, chunks))
    return np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts])


_default: Oracle | None = None


def get() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default
