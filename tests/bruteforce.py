"""Independent brute-force reference for tiny inputs (numpy, written apart from the oracle).

Used only to check the C oracle on small shapes.  It restates the same
definitions with different code: numpy float32 element-wise arithmetic for the
quantization decisions (IEEE binary32 divide and multiply, np.rint = round half
to even), numpy int64 products for the integer stage, and float64 for the
output.  Page: "A Gentle Introduction to 8-bit Matrix Multiplication for
transformers at scale", sections "absmax quantization", "LLM.int8() summary",
"inside the MatMul" and "Usage".
"""
from __future__ import annotations

import numpy as np


def widen(bits: np.ndarray, dtype: int) -> np.ndarray:
    bits = np.asarray(bits, dtype=np.uint16)
    if dtype == 0:
        return bits.view(np.float16).astype(np.float32)
    return (bits.astype(np.uint32) << 16).view(np.float32)


def absmax_quantize_rows(A: np.ndarray, keep: np.ndarray | None = None):
    """Row-wise absmax quantization of float32 A [R, K] over the kept columns.

    Returns (q int8 [R, K], absmax float32 [R]).  Columns not kept are 0.
    """
    R, K = A.shape
    keep = np.ones(K, dtype=bool) if keep is None else keep
    q = np.zeros((R, K), dtype=np.int8)
    amax = np.zeros(R, dtype=np.float32)
    for r in range(R):
        vals = np.abs(A[r, keep])
        a = np.float32(vals.max()) if vals.size else np.float32(0)
        amax[r] = a
        if a == 0:
            continue
        s = np.float32(127) / a                   # binary32 division
        p = (A[r] * s).astype(np.float32)          # binary32 multiply
        v = np.clip(np.rint(p), -127, 127).astype(np.int8)
        q[r] = np.where(keep, v, 0)
    return q, amax


def forward(X: np.ndarray, W: np.ndarray, dtype: int, threshold: float, bias=None):
    x = widen(X, dtype)
    w = widen(W, dtype)
    M, K = x.shape
    CB, SCB = absmax_quantize_rows(w)
    colmax = np.abs(x).max(axis=0) if M else np.zeros(K, np.float32)
    outlier = (colmax >= np.float32(threshold)) if M else np.zeros(K, bool)
    idx = np.nonzero(outlier)[0].astype(np.int32)
    CA, SCA = absmax_quantize_rows(x, keep=~outlier)
    XO = np.asarray(X, dtype=np.uint16)[:, idx]
    C = CA.astype(np.int64) @ CB.astype(np.int64).T
    assert np.abs(C).max(initial=0) < 2**31
    Wdq = CB.astype(np.float64) * SCB.astype(np.float64)[:, None] / 127.0
    Y = C.astype(np.float64) * np.outer(SCA.astype(np.float64), SCB.astype(np.float64)) / 16129.0
    Y = Y + x[:, idx].astype(np.float64) @ Wdq[:, idx].T
    if bias is not None:
        Y = Y + widen(np.asarray(bias), dtype).astype(np.float64)[None, :]
    return dict(CB=CB, SCB=SCB, CA=CA, SCA=SCA, idx=idx, XO=XO, C=C.astype(np.int32), Y=Y)
