"""Synthetic accuracy ablation of the quantization schemes.

    python -m int8_quantized_matmul_row_amd.ablation [--M 256 --N 2048 --K 2048]

Compares, on seeded synthetic layers, the error of Y = X . W^T against an
exact reference (float64 on the host, from the same 16-bit X and W) for
  * per-tensor absmax: one scale for all of X and one for all of W
    ("A Gentle Introduction to 8-bit Matrix Multiplication for transformers at
    scale", section "absmax quantization");
  * vector-wise absmax: one scale per token row of X and per output channel of
    W (same page, section "inside the MatMul") -- LLM.int8() with no outlier
    columns (threshold +inf);
  * LLM.int8(): vector-wise int8 plus 16-bit outlier columns at thresholds
    2, 4, 6 (the pages' value) and 8 (same page, section "LLM.int8() summary");
  * the FP8 variant (E4M3 codes in place of int8, the 8-bit floating-point
    type the zhichai.top summary lists as future work) at threshold 6, and
    FP8 vector-wise (threshold +inf).
across outlier-column densities 0, 0.1% (the density the pages report for
large models: "LLM.int8() : Multiplication matricielle à 8 bits pour les
Transformers à grande échelle", abstract), 1% and 5%.  Every scheme runs in
libllmint8's kernels; the reference product is the only host arithmetic.

Prints one JSON line per (density, scheme) and a markdown table.
"""
from __future__ import annotations

import argparse
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _widen(bits, dtype):
    import synth
    return synth.bits_to_f32(bits, dtype).astype(np.float64)


def run(M=256, N=2048, K=2048, densities=(0.0, 0.001, 0.01, 0.05), thresholds=(2.0, 4.0, 6.0, 8.0),
        seed=0, device="cuda:0", fp8=True):
    """Returns a list of dicts: density, scheme, threshold, n_out, rel_fro, max_rel."""
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    import torch
    import synth
    import int8_quantized_matmul_row_amd as pkg
    dev = torch.device(device)
    rows = []
    for f in densities:
        n_cols = int(round(f * K))
        wl = synth.make_random(M, N, K, synth.F16, seed=seed, n_outlier_cols=n_cols,
                               lo=8.0, hi=60.0, w_sigma=0.02)
        Yref = _widen(wl.X, synth.F16) @ _widen(wl.W, synth.F16).T
        scale = np.abs(Yref).max()
        fro = np.linalg.norm(Yref)
        X = torch.from_numpy(wl.X.view(np.int16)).to(dev).view(torch.float16)
        W = torch.from_numpy(wl.W.view(np.int16)).to(dev).view(torch.float16)

        def record(name, t, Y, n_out):
            y = Y.float().cpu().numpy().astype(np.float64)
            err = y - Yref
            rows.append(dict(density=f, outlier_cols=n_cols, scheme=name, threshold=t, n_out=n_out,
                             rel_fro=float(np.linalg.norm(err) / fro),
                             max_rel=float(np.abs(err).max() / scale)))

        Qx, sx = pkg.quantize_tensor(X)
        Qw, sw = pkg.quantize_tensor(W)
        record("per-tensor absmax", None, pkg.matmul_codes(Qx, sx, Qw, sw, X.dtype), 0)
        CB, SCB = pkg.quantize_weight(W)
        for t in (float("inf"),) + tuple(thresholds):
            Y, q = pkg.linear(X, CB, SCB, threshold=t)
            name = "vector-wise" if t == float("inf") else "LLM.int8()"
            record(name, None if t == float("inf") else t, Y, int(q.n_out.item()))
        if fp8:
            CB8, SCB8 = pkg.quantize_weight_fp8(W)
            for t in (float("inf"), 6.0):
                Y, q = pkg.linear_fp8(X, CB8, SCB8, threshold=t)
                name = "FP8 vector-wise" if t == float("inf") else "FP8 LLM.int8()"
                record(name, None if t == float("inf") else t, Y, int(q.n_out.item()))
    return rows


def table(rows) -> str:
    out = ["| outlier columns | scheme | threshold | outliers used | rel. Frobenius error | max error / max abs(Y) |",
           "|---|---|---|---|---|---|"]
    for r in rows:
        t = "-" if r["threshold"] is None else f"{r['threshold']:g}"
        out.append(f"| {r['outlier_cols']} ({100 * r['density']:g}%) | {r['scheme']} | {t} | "
                   f"{r['n_out']} | {r['rel_fro']:.3e} | {r['max_rel']:.3e} |")
    return "\n".join(out)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--M", type=int, default=256)
    ap.add_argument("--N", type=int, default=2048)
    ap.add_argument("--K", type=int, default=2048)
    ap.add_argument("--seed", type=int, default=0)
    args = ap.parse_args()
    rows = run(args.M, args.N, args.K, seed=args.seed)
    for r in rows:
        print(json.dumps(r), flush=True)
    print(f"\nX fp16 [{args.M}x{args.K}] ~N(0,1), outlier columns +-U(8,60); "
          f"W fp16 [{args.N}x{args.K}] ~N(0,0.02); seed {args.seed}\n")
    print(table(rows), flush=True)


if __name__ == "__main__":
    main()
