"""Seeded synthetic inputs for the LLM.int8() decomposition matmul.

This module is shared by the CPU oracle's tests and by the GPU path's tests and
benchmark.  It only draws random numbers and converts them to 16-bit bit
patterns; it holds none of the method's arithmetic (no absmax, no threshold
test, no quantization, no product).

Workloads (all Y = X.W^T with X [M,K] tokens x features, W [N,K] nn.Linear
layout, threshold 6.0 -- the value at which the pages extract outliers, "A Gentle
Introduction to 8-bit Matrix Multiplication for transformers at scale", section
"inside the MatMul"):

  tiny      X fp16 [16 x 1024] ~N(0,1), feature columns 7 and 500 set to +-20
            (sign of the body draw kept); W fp16 [1024 x 1024] ~N(0,0.02); no bias
  decode    X fp16 [8 x 4096] ~N(0,1), 4 outlier columns (0.1%) |x|~U(8,60);
            W fp16 [4096 x 4096] ~N(0,0.02); no bias
  prefill   X fp16 [2048 x 4096], 4 outlier columns U(8,60); W fp16
            [16384 x 4096] ~N(0,0.02); bias fp16 ~N(0,0.01)
  bloom_up  X bf16 [512 x 14336], 14 outlier columns U(6,80); W bf16
            [57344 x 14336] ~N(0,0.01); no bias
  bloom_down X bf16 [512 x 57344] drawn independently, 57 outlier columns
            U(6,80); W bf16 [14336 x 57344] ~N(0,0.01); no bias
  sweep_<f> X fp16 [4096 x 8192], outlier fraction f in {0, 0.1, 1, 5}% ->
            {0, 8, 82, 410} columns U(8,60); W fp16 [28672 x 8192] ~N(0,0.02)

The ~0.1% outlier-dimension density follows the pages ("LLM.int8() : Multiplication
matricielle a 8 bits pour les Transformers a grande echelle", abstract: more than
99.9% of values stay in 8-bit; the zhichai.top LLM.int8() summary, section on
emergent outlier features: about 0.1% of feature dimensions).

Recipe: numpy.random.default_rng([seed, stream]); streams 0 = X body,
1 = X outlier columns / signs / magnitudes, 2 = W, 3 = bias, 4 = bloom_down X
body, 5 = bloom_down outlier columns.  Normal draws are float32
(standard_normal(dtype=float32), drawn in row chunks of the same stream, which
gives the same sequence as one draw), scaled by sigma in float32, then rounded
to fp16 (numpy astype, round-to-nearest-even) or bf16 (round-to-nearest-even
on the float32 bits).  Outlier columns: rng.choice(K, n, replace=False), each
entry +-U(lo, hi) with an equiprobable sign.
"""
from __future__ import annotations

import dataclasses
import numpy as np

F16 = 0
BF16 = 1
DTYPE_NAMES = {F16: "fp16", BF16: "bf16"}

_CHUNK_ELEMS = 1 << 24  # rows are drawn in chunks of about this many elements


def f32_to_f16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> IEEE binary16 bit patterns (round to nearest even)."""
    return np.ascontiguousarray(a, dtype=np.float32).astype(np.float16).view(np.uint16)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (round to nearest even; finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    rounding = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + rounding) >> 16).astype(np.uint16)


def to_bits(a: np.ndarray, dtype: int) -> np.ndarray:
    return f32_to_f16_bits(a) if dtype == F16 else f32_to_bf16_bits(a)


def bits_to_f32(b: np.ndarray, dtype: int) -> np.ndarray:
    """16-bit bit patterns -> float32 (exact).  Convenience for tests and plots."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    if dtype == F16:
        return b.view(np.float16).astype(np.float32)
    return (b.astype(np.uint32) << 16).view(np.float32)


def normal_bits(seed: int, stream: int, rows: int, cols: int, sigma: float, dtype: int) -> np.ndarray:
    """[rows, cols] 16-bit bit patterns of sigma * N(0,1), drawn in row chunks."""
    rng = np.random.default_rng([seed, stream])
    out = np.empty((rows, cols), dtype=np.uint16)
    step = max(1, _CHUNK_ELEMS // max(cols, 1))
    sig = np.float32(sigma)
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        z = rng.standard_normal((r1 - r0, cols), dtype=np.float32)
        if sigma != 1.0:
            z *= sig
        out[r0:r1] = to_bits(z, dtype)
    return out


def plant_outlier_columns(xbits: np.ndarray, dtype: int, seed: int, stream: int,
                          n_cols: int, lo: float, hi: float) -> np.ndarray:
    """Overwrite n_cols random feature columns of X with +-U(lo, hi) entries.

    Returns the planted column indices (ascending).  The oracle, not this
    function, decides which columns are outliers.
    """
    M, K = xbits.shape
    if n_cols == 0:
        return np.zeros(0, dtype=np.int64)
    rng = np.random.default_rng([seed, stream])
    cols = np.sort(rng.choice(K, n_cols, replace=False))
    mag = rng.uniform(lo, hi, size=(M, n_cols)).astype(np.float32)
    sign = np.where(rng.random((M, n_cols)) < 0.5, np.float32(-1), np.float32(1))
    xbits[:, cols] = to_bits(mag * sign, dtype)
    return cols.astype(np.int64)


@dataclasses.dataclass
class Workload:
    name: str
    dtype: int          # F16 or BF16; X, W, bias and Y share it
    M: int
    N: int
    K: int
    threshold: float
    X: np.ndarray       # uint16 [M, K]
    W: np.ndarray       # uint16 [N, K]
    bias: np.ndarray | None  # uint16 [N] or None
    planted_cols: np.ndarray

    @property
    def ops(self) -> int:
        return 2 * self.M * self.N * self.K


# name -> (dtype, M, N, K, outlier cols, lo, hi, w sigma, bias sigma, x stream, xo stream)
_SPECS = {
    "tiny": (F16, 16, 1024, 1024, None, 20.0, 20.0, 0.02, None, 0, 1),
    "decode": (F16, 8, 4096, 4096, 4, 8.0, 60.0, 0.02, None, 0, 1),
    "prefill": (F16, 2048, 16384, 4096, 4, 8.0, 60.0, 0.02, 0.01, 0, 1),
    "bloom_up": (BF16, 512, 57344, 14336, 14, 6.0, 80.0, 0.01, None, 0, 1),
    "bloom_down": (BF16, 512, 14336, 57344, 57, 6.0, 80.0, 0.01, None, 4, 5),
    "sweep_0": (F16, 4096, 28672, 8192, 0, 8.0, 60.0, 0.02, None, 0, 1),
    "sweep_0.1": (F16, 4096, 28672, 8192, 8, 8.0, 60.0, 0.02, None, 0, 1),
    "sweep_1": (F16, 4096, 28672, 8192, 82, 8.0, 60.0, 0.02, None, 0, 1),
    "sweep_5": (F16, 4096, 28672, 8192, 410, 8.0, 60.0, 0.02, None, 0, 1),
    # batched decode: 32 tokens through the sweep's layer (the weight-streaming
    # product)
    "batch_32": (F16, 32, 28672, 8192, 4, 8.0, 60.0, 0.02, None, 0, 1),
}

WORKLOADS = tuple(_SPECS)


def workload_shape(name: str):
    dt, M, N, K = _SPECS[name][:4]
    return dt, M, N, K


def make_workload(name: str, seed: int = 0, with_weight: bool = True,
                  threshold: float = 6.0) -> Workload:
    """Build one named workload.  with_weight=False skips W (and bias)."""
    dt, M, N, K, ncols, lo, hi, wsig, bsig, xs, xos = _SPECS[name]
    X = normal_bits(seed, xs, M, K, 1.0, dt)
    if name == "tiny":
        # Columns 7 and 500 scaled to magnitude 20, keeping the body's sign.
        cols = np.array([7, 500], dtype=np.int64)
        body = bits_to_f32(X[:, cols], dt)
        X[:, cols] = to_bits(np.where(body < 0, np.float32(-20), np.float32(20)), dt)
        planted = cols
    else:
        planted = plant_outlier_columns(X, dt, seed, xos, ncols, lo, hi)
    W = normal_bits(seed, 2, N, K, wsig, dt) if with_weight else None
    bias = None
    if with_weight and bsig is not None:
        bias = normal_bits(seed, 3, 1, N, bsig, dt).reshape(N)
    return Workload(name, dt, M, N, K, threshold, X, W, bias, planted)


def make_random(M: int, N: int, K: int, dtype: int = F16, seed: int = 0,
                n_outlier_cols: int = 0, lo: float = 8.0, hi: float = 60.0,
                w_sigma: float = 0.02, bias_sigma: float | None = None,
                threshold: float = 6.0) -> Workload:
    """An arbitrary-shape workload with the same recipe (for tests)."""
    X = normal_bits(seed, 0, M, K, 1.0, dtype)
    planted = plant_outlier_columns(X, dtype, seed, 1, n_outlier_cols, lo, hi)
    W = normal_bits(seed, 2, N, K, w_sigma, dtype)
    bias = None if bias_sigma is None else normal_bits(seed, 3, 1, N, bias_sigma, dtype).reshape(N)
    return Workload(f"random_{M}x{N}x{K}", dtype, M, N, K, threshold, X, W, bias, planted)
