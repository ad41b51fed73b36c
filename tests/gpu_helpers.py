"""Helpers for the GPU parity tests: run the HIP path through the C-ABI on a
workload and compare every stage with the CPU oracle."""
from __future__ import annotations

import os
import sys

import numpy as np

import synth

Y_GATE = 1e-2        # max |dY| <= 1e-2 * max |Y_ref|
Y_REL = 1e-4         # per element: |dY| <= ulp16(|Y_ref|) + 1e-4 * max |Y_ref|


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def ulp16(y: np.ndarray, dtype: int) -> np.ndarray:
    """Spacing of the 16-bit format at |y| (the output's rounding step)."""
    a = np.abs(y).astype(np.float64)
    if dtype == synth.F16:
        return np.spacing(a.astype(np.float16)).astype(np.float64)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return 2.0 ** (e - 7)


def to_torch(bits: np.ndarray, dtype: int, device):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    t = t.view(torch.float16 if dtype == synth.F16 else torch.bfloat16)
    return t.to(device)


def bits_of(t) -> np.ndarray:
    import torch
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def run_gpu(wl, threshold=None, want_C=True, weight=None, device="cuda:0"):
    """Full HIP path on workload wl.  Returns numpy arrays of every stage."""
    import torch
    import int8_quantized_matmul_row_amd as pkg
    t = wl.threshold if threshold is None else threshold
    dev = torch.device(device)
    X = to_torch(wl.X, wl.dtype, dev)
    if weight is None:
        W = to_torch(wl.W, wl.dtype, dev)
        CB, SCB = pkg.quantize_weight(W)
        del W
    else:
        CB, SCB = weight
    bias = None if wl.bias is None else to_torch(wl.bias, wl.dtype, dev)
    q = pkg.quantize_act(X, t)
    C = torch.empty((wl.M, wl.N), dtype=torch.int32, device=dev) if want_C else None
    Y = pkg.matmul(q, CB, SCB, bias=bias, C_i32=C)
    torch.cuda.synchronize()
    n_out = int(q.n_out.item())
    n_pad = (n_out + 31) // 32 * 32
    out = dict(
        CA=q.CA.cpu().numpy(), SCA=q.SCA.cpu().numpy(),
        idx=q.idx[:n_out].cpu().numpy(), n_out=n_out,
        XO=bits_of(q.XO[:wl.M * n_pad]).reshape(wl.M, n_pad),
        Y=bits_of(Y), weight=(CB, SCB), C_dev=C, Y_dev=Y)
    if weight is None:
        out["CB"] = CB.cpu().numpy()
        out["SCB"] = SCB.cpu().numpy()
    return out


def run_gpu_linear(wl, threshold=None, weight=None, device="cuda:0", workspace=None):
    """The one-call forward (llmint8_linear) on workload wl; same dict as run_gpu."""
    import torch
    import int8_quantized_matmul_row_amd as pkg
    t = wl.threshold if threshold is None else threshold
    dev = torch.device(device)
    X = to_torch(wl.X, wl.dtype, dev)
    if weight is None:
        CB, SCB = pkg.quantize_weight(to_torch(wl.W, wl.dtype, dev))
    else:
        CB, SCB = weight
    bias = None if wl.bias is None else to_torch(wl.bias, wl.dtype, dev)
    C = torch.empty((wl.M, wl.N), dtype=torch.int32, device=dev)
    Y, q = pkg.linear(X, CB, SCB, bias=bias, threshold=t, C_i32=C, workspace=workspace)
    torch.cuda.synchronize()
    n_out = int(q.n_out.item())
    n_pad = (n_out + 31) // 32 * 32
    out = dict(
        CA=q.CA.cpu().numpy(), SCA=q.SCA.cpu().numpy(),
        idx=q.idx[:n_out].cpu().numpy(), n_out=n_out,
        XO=bits_of(q.XO[:wl.M * n_pad]).reshape(wl.M, n_pad),
        Y=bits_of(Y), weight=(CB, SCB), C_dev=C, Y_dev=Y)
    if weight is None:
        out["CB"] = CB.cpu().numpy()
        out["SCB"] = SCB.cpu().numpy()
    return out


def check_y(Ybits: np.ndarray, Yref: np.ndarray, dtype: int, label: str):
    y = synth.bits_to_f32(Ybits, dtype).astype(np.float64)
    assert np.all(np.isfinite(y)), label
    err = np.abs(y - Yref)
    scale = np.abs(Yref).max()
    gate = err.max() <= Y_GATE * scale
    bound = ulp16(Yref, dtype) + Y_REL * scale
    bad = err > bound
    assert gate, f"{label}: max|dY| {err.max():.4g} > 1e-2 * {scale:.4g}"
    assert not bad.any(), (f"{label}: {bad.sum()} elements beyond ulp16 + 1e-4*max|Y|, "
                           f"worst {err[bad].max():.4g}")
    return float(err.max()), float(scale)


def compare(wl, g, ref, rows=None, label=""):
    """Bit-exact integer stages, tolerance on Y.  ref from oracle.forward."""
    label = label or wl.name
    if "CB" in g:
        assert np.array_equal(g["CB"], ref["CB"]), f"{label}: CB"
        assert np.array_equal(g["SCB"], ref["SCB"]), f"{label}: SCB"
    assert g["n_out"] == len(ref["idx"]), f"{label}: n_out {g['n_out']} vs {len(ref['idx'])}"
    assert np.array_equal(g["idx"], ref["idx"]), f"{label}: outlier index list"
    assert np.array_equal(g["SCA"], ref["SCA"]), f"{label}: SCA"
    assert np.array_equal(g["CA"], ref["CA"]), f"{label}: CA"
    n_out = g["n_out"]
    assert np.array_equal(g["XO"][:, :n_out], ref["XO"]), f"{label}: XO"
    assert not g["XO"][:, n_out:].any(), f"{label}: XO padding"
    sel = slice(None) if rows is None else rows
    if g.get("C_dev") is not None:
        import torch
        C = g["C_dev"] if rows is None else g["C_dev"][torch.as_tensor(rows, device=g["C_dev"].device)]
        assert np.array_equal(C.cpu().numpy(), ref["C"]), f"{label}: int32 accumulators"
    return check_y(g["Y"][sel], ref["Y"], wl.dtype, label)


def sample_rows(M, n, seed=0):
    rng = np.random.default_rng([seed, 99])
    rows = {0, M - 1}
    while len(rows) < min(n, M):
        rows.add(int(rng.integers(0, M)))
    return np.array(sorted(rows), dtype=np.int64)


def host_threads() -> int:
    """Threads for the oracle's row loops: this process's CPUs, at most 16 (a
    GPU host's share)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def oracle_forward(orc, wl, threshold, weight, rows=None):
    """orc.forward's dict, with the product and output rows spread over
    host_threads() threads (the oracle's own per-row functions; the same result
    for any thread count).  rows=None: every row."""
    import oracle
    CB, SCB = weight
    act = orc.quantize_act(wl.X, wl.dtype, threshold)
    rows = np.arange(wl.M, dtype=np.int64) if rows is None else rows
    C, Y = oracle.forward_rows_threaded(orc, act, weight, wl.X, wl.dtype, wl.bias, rows,
                                        host_threads())
    CA, SCA, idx, XO = act
    return dict(CB=CB, SCB=SCB, CA=CA, SCA=SCA, idx=idx, XO=XO, C=C, Y=Y)
