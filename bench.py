"""Benchmark of the LLM.int8() decomposition matmul on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config decode|prefill|...]
                    [--variant int8|fp8]

A step is one forward of the layer on resident inputs through llmint8_linear:
outlier columns, row scales and int8 activations (llmint8_quantize_act's
results), then the int8 MFMA product, dequantization, 16-bit outlier product
and bias (llmint8_matmul's).  For a handful of tokens this is one fused kernel;
otherwise the activation kernels then the tiled GEMM.  Weight quantization runs
once per weight, at load time, and is reported separately.

Prints one JSON line.  value = effective TOPS = 2*M*N*K / step time.  The
dominant kernel (the matmul) is also timed on its own with HIP events bound to
its dispatch, and placed against its roofline: HBM bandwidth for small-M
(decode) shapes, int8 MFMA throughput otherwise.  Distinct copies of the int8
weight are rotated, more than 512 MiB in total, so each step streams its weight
from HBM rather than from the 256 MiB Infinity Cache.

--variant fp8 runs the FP8 (E4M3) variant of the same decomposition
(llmint8_linear_fp8: the activation kernels, then the fp8 GEMM) and prices its
GEMM against the dense fp8 MFMA peak or HBM.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "LLM.int8 matmul effective TOPS (2MNK/s) + % of int8-MFMA / HBM roofline"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
INT8_PEAK_TOPS = 5000.0      # MI355X dense int8 MFMA
FP8_PEAK_TFLOPS = 5000.0     # MI355X dense fp8 MFMA
ROTATE_BYTES = 512 << 20     # > 2x the Infinity Cache
# the largest workload that fits one GPU: 4096 x 28672 x 8192 fp16 with 0.1% outlier columns
DEFAULT_CONFIG = "sweep_0.1"
KERNEL_SOURCES = {
    "decode": ["int8_quantized_matmul_row_amd/csrc/linear_decode.hip",
               "int8_quantized_matmul_row_amd/csrc/common.h"],
    "fused": ["int8_quantized_matmul_row_amd/csrc/linear_small_m.hip",
              "int8_quantized_matmul_row_amd/csrc/common.h"],
    "small_m": ["int8_quantized_matmul_row_amd/csrc/gemm_small_m.hip",
                "int8_quantized_matmul_row_amd/csrc/common.h"],
    "tiled": ["int8_quantized_matmul_row_amd/csrc/gemm_tiled.hip",
              "int8_quantized_matmul_row_amd/csrc/common.h"],
}


KERNEL_NAMES = {"decode": "linear_decode_kernel", "fused": "linear_small_m_kernel", "small_m": "gemm_small_m_kernel",
                "tiled": "gemm_tiled_kernel"}


def small_m_product(M, N, K):
    """Whether the product takes the weight-streaming kernel (the library's
    rule): up to 16 token rows always; up to 64 when M * N * K is at most 6e9
    or the streaming grid is one round of the chip: up to 32 rows at most 512
    workgroups (of 64 channels when N >= 16384, else of 16), above that at
    most 256 workgroups of 64 channels."""
    if M <= 16:
        return True
    if M > 64 or N is None:
        return False
    wide = N >= 64 * 256
    if M <= 32:
        one_round = -(-N // (64 if wide else 16)) <= 512
    else:
        one_round = wide and -(-N // 64) <= 256
    return M * N * K <= 6_000_000_000 or one_round


def kernel_family(M, K, variant="int8", N=None):
    """The kernel that carries the product in llmint8_linear (or
    llmint8_linear_fp8, which has the fused decode kernel but not the other
    fused small-M one) for this shape."""
    if 1 <= M <= 8 and M * K <= 32768 and K <= 8192:
        return "decode"
    if variant == "fp8":
        return "small_m" if small_m_product(M, N, K) else "tiled"
    if 1 <= M <= 16 and M * K <= 65536 and K <= 8192:
        return "fused"
    return "small_m" if small_m_product(M, N, K) else "tiled"


def source_hash(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(family, M, N, K, n_out, has_bias):
    """Bytes the kernel must move.  GEMM kernels: CB, SCB, CA, SCA, the 16-bit
    outlier activations (n_pad columns) and their index list, bias, Y.  The fused
    kernel reads X instead of CA, and also writes the activation outputs (CA,
    SCA, index list, count, XO)."""
    n_pad = (n_out + 31) // 32 * 32
    common = N * K + 4 * N + (2 * N if has_bias else 0) + 2 * M * N
    act_out = M * K + 4 * M + 2 * M * n_pad + 4 * n_out
    if family in ("decode", "fused"):
        return common + 2 * M * K + act_out + 4
    return common + act_out


class Hip:
    """The few HIP runtime calls the benchmark makes itself (events)."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]

    def event(self):
        ev = ctypes.c_void_p()
        rc = self.lib.hipEventCreate(ctypes.byref(ev))
        if rc != 0:
            raise RuntimeError(f"hipEventCreate failed: {rc}")
        return ev.value

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        rc = self.lib.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b))
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {rc}")
        return ms.value


def load_traffic(config, family, variant="int8", threshold=None):
    """HBM traffic per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source (and at the threshold asked for, when
    it is not the workload's own); otherwise None."""
    suffix = ("" if variant == "int8" else f"_{variant}") + ("" if threshold is None else f"_t{threshold:g}")
    path = os.path.join(ROOT, "profiles", f"traffic_{config}{suffix}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_sha256") != source_hash(KERNEL_SOURCES[family]):
        return None
    return t.get("hbm_bytes_per_launch")


def host_cores():
    """Host cores this process may use: its CPU affinity, capped by
    OMP_NUM_THREADS when that is set (the GPU host's share of its CPUs)."""
    n = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return max(1, n)


def cpu_baseline(wl, variant="int8", budget_1core_s=8.0, budget_ncore_s=10.0):
    """The CPU oracle, as it stands, on a bounded sample of the same step.

    The step is quantize_act over all M rows (single-threaded: the outlier set
    couples the rows) plus the product and output of every row.  Two legs:
    1 core, rows taken in a fixed random order until the budget is spent; and
    the same per-row functions on every host core (`host_cores()` threads, each
    on a contiguous chunk of an evenly spaced row sample sized to the budget).
    Each leg's time is t(quantize_act) + t(rows) * M / rows.  Returns
    (all-cores leg, 1-core leg)."""
    import numpy as np
    import oracle
    orc = oracle.get()
    fp8 = variant == "fp8"
    weight = (orc.quantize_weight_fp8 if fp8 else orc.quantize_weight)(wl.W, wl.dtype)
    M, N, K = wl.M, wl.N, wl.K
    ops = 2 * M * N * K
    t0 = time.perf_counter()
    act = (orc.quantize_act_fp8 if fp8 else orc.quantize_act)(wl.X, wl.dtype, wl.threshold)
    t_act = time.perf_counter() - t0

    # 1 core: rows 0 and M-1, then the others in a fixed random order, cycling
    perm = np.random.default_rng(0).permutation(M)
    uniq = [0, M - 1] + [int(r) for r in perm if r not in (0, M - 1)] if M > 1 else [0]
    done, t0 = 0, time.perf_counter()
    while True:  # chunks of up to 8 rows per call
        r = np.array([uniq[(done + i) % M] for i in range(min(8, M))], dtype=np.int64)
        oracle.forward_rows_threaded(orc, act, weight, wl.X, wl.dtype, wl.bias, r, 1, fp8=fp8)
        done += len(r)
        el = time.perf_counter() - t0
        if el >= budget_1core_s:
            break
    rate1 = done / el
    step1 = t_act + M / rate1
    one = {"value": round(ops / step1 / 1e12, 6), "unit": "TOPS", "cores": 1, "kind": "oracle",
           "sample": (f"quantize_act on all {M} rows ({t_act:.2f} s) + {done} rows of the product "
                      f"and output on 1 core ({el:.1f} s), extrapolated to {M} rows"
                      + (f" (the {M} rows cycled)" if done > M else "")),
           "ms_per_step": round(step1 * 1e3, 3)}

    # every core: a sample sized to the budget, split into per-thread chunks
    cores = host_cores()
    n_rows = int(min(M, max(1, rate1 * cores * budget_ncore_s)))
    threads = min(cores, n_rows)
    rows = np.unique(np.linspace(0, M - 1, n_rows).round().astype(np.int64))
    passes, t0 = 0, time.perf_counter()
    while True:  # whole passes over the sample until the budget is spent
        oracle.forward_rows_threaded(orc, act, weight, wl.X, wl.dtype, wl.bias, rows, threads,
                                     fp8=fp8)
        passes += 1
        el_n = time.perf_counter() - t0
        if el_n >= budget_ncore_s / 2:
            break
    t_rows = el_n / passes
    stepn = t_act + t_rows * M / len(rows)
    full = len(rows) == M
    alln = {"value": round(ops / stepn / 1e12, 6), "unit": "TOPS", "cores": threads,
            "kind": "oracle",
            "sample": (f"quantize_act on all {M} rows ({t_act:.2f} s, 1 thread) + the product and "
                       f"output of {'all ' if full else ''}{len(rows)}"
                       f"{'' if full else ' evenly spaced'} rows on {threads} threads "
                       f"({t_rows:.3g} s per pass, {passes} passes)"
                       f"{'' if full else f', extrapolated to {M} rows'}"),
            "ms_per_step": round(stepn * 1e3, 3)}
    return alln, one


def calibrate_copy(torch, dev, nbytes, launches):
    """A plain copy of known size: each launch reads and writes nbytes once."""
    src = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(launches):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "copy", "bytes_read_per_launch": nbytes,
                      "bytes_written_per_launch": nbytes, "launches": launches}), flush=True)


def measured_ceiling(torch, pkg, dev, bound, fp8):
    """The ceiling measured on this device beside the published peak.  HBM:
    a plain 1 GiB device-to-device copy (its read and its write counted).
    MFMA: the library's sustained-rate loop (llmint8_peak_mfma) on random
    codes, every CU busy.  Median of 5 timed launches after 2 warm-ups."""
    stream = torch.cuda.current_stream()
    times = []
    if bound == "hbm":
        nbytes = 1 << 30
        src = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)
        dst = torch.empty_like(src)
        for i in range(7):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            dst.copy_(src)
            e1.record(stream)
            torch.cuda.synchronize()
            if i >= 2:
                times.append(e0.elapsed_time(e1) * 1e-3)
        t = sorted(times)[len(times) // 2]
        del src, dst
        return {"value": round(2 * nbytes / t / 1e9, 1), "unit": "GB/s",
                "how": "device-to-device copy of 1 GiB, read + write bytes / time"}
    g = torch.Generator(device="cpu").manual_seed(7)
    codes = torch.randint(-128, 128, (262144,), dtype=torch.int8, generator=g)
    if fp8:  # finite E4M3 codes only (0x7f and 0xff are NaN)
        codes[(codes == 127) | (codes == -1)] = 1
    operands = codes.to(dev)
    blocks, iters = 1024, 512
    sink = torch.empty(blocks * 256, dtype=torch.int32, device=dev)
    for i in range(7):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        pkg.llmint8_peak_mfma(1 if fp8 else 0, operands.data_ptr(), operands.numel(), sink.data_ptr(),
                              sink.numel() * 4, blocks, iters, stream.cuda_stream)
        e1.record(stream)
        torch.cuda.synchronize()
        if i >= 2:
            times.append(e0.elapsed_time(e1) * 1e-3)
    t = sorted(times)[len(times) // 2]
    ops = blocks * 16 * iters * (131072 if fp8 else 65536)
    return {"value": round(ops / t / 1e12, 1), "unit": "TFLOP/s" if fp8 else "TOP/s",
            "how": ("v_mfma_scale_f32_32x32x64_f8f6f4" if fp8 else "v_mfma_i32_32x32x32_i8")
                   + " back to back on random codes, 1024 workgroups x 4 waves"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default=DEFAULT_CONFIG)
    ap.add_argument("--threshold", type=float, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--variant", choices=("int8", "fp8"), default="int8",
                    help="int8 codes (the method) or the FP8 (E4M3) variant")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (steps times), "
                         "the reference kernel for scaling HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the path runs on a single MI355X).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import int8_quantized_matmul_row_amd as pkg
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.calibrate_copy:
        calibrate_copy(torch, dev, args.calibrate_copy << 20, args.steps)
        return
    hip = Hip()
    wl = synth.make_workload(args.config)
    if args.threshold is not None:
        wl.threshold = args.threshold
    M, N, K = wl.M, wl.N, wl.K
    dt_t = torch.float16 if wl.dtype == synth.F16 else torch.bfloat16

    def dev16(bits):
        return torch.from_numpy(bits.view(np.int16)).to(dev).view(dt_t)

    X = dev16(wl.X)
    W = dev16(wl.W)
    bias = None if wl.bias is None else dev16(wl.bias)

    fp8 = args.variant == "fp8"
    quantize_w = pkg.quantize_weight_fp8 if fp8 else pkg.quantize_weight

    # ---- one-time weight quantization (S1), timed on its own ---------------
    CB0 = torch.empty((N, K), dtype=torch.uint8 if fp8 else torch.int8, device=dev)
    SCB0 = torch.empty((N,), dtype=torch.float32, device=dev)
    for _ in range(3):
        quantize_w(W, out=(CB0, SCB0))
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 10
    e0.record()
    for _ in range(reps):
        quantize_w(W, out=(CB0, SCB0))
    e1.record()
    torch.cuda.synchronize()
    wq_ms = e0.elapsed_time(e1) / reps
    wq_bytes = 2 * N * K + N * K + 4 * N
    del W

    # ---- resident buffers: rotated weight copies, activations, outputs -------
    n_copies = max(1, -(-ROTATE_BYTES // (N * K)))
    weights = [(CB0, SCB0)] + [(CB0.clone(), SCB0.clone()) for _ in range(n_copies - 1)]
    q = pkg.alloc_act(M, K, dt_t, dev, fp8=fp8)
    ws = (pkg.linear_fp8_workspace if fp8 else pkg.linear_workspace)(M, N, K, dev)
    linear_fn = pkg.llmint8_linear_fp8 if fp8 else pkg.llmint8_linear
    linear_prof = pkg.llmint8_linear_fp8_profiled if fp8 else pkg.llmint8_linear_profiled
    Y = torch.empty((M, N), dtype=dt_t, device=dev)
    stream = torch.cuda.Stream()
    s_ptr = stream.cuda_stream

    def step(i, ev=None):
        CB, SCB = weights[i % n_copies]
        a = (X.data_ptr(), wl.dtype, M, N, K, wl.threshold, CB.data_ptr(), SCB.data_ptr(),
             None if bias is None else bias.data_ptr(), Y.data_ptr(), q.CA.data_ptr(),
             q.SCA.data_ptr(), q.idx.data_ptr(), q.n_out.data_ptr(), q.XO.data_ptr(), None,
             ws[0].data_ptr(), ws[1], s_ptr)
        if ev is None:
            linear_fn(*a)
        else:
            linear_prof(*a, ev[0], ev[1])

    # ---- warmup ---------------------------------------------------------------
    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            step(i)
    torch.cuda.synchronize()
    n_out = int(q.n_out.item())

    # The timed region replays one graph of exactly `steps` steps, step i on
    # weight copy i % n_copies (a decode step is a few microseconds of GPU
    # work, far below the cost of launching it from Python).  The graph is
    # replayed once untimed first.
    steps = args.steps
    graph = None
    if not args.no_graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            for i in range(steps):
                step(i)
        graph.replay()
    torch.cuda.synchronize()

    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        g0.record(stream)
        if graph is not None:
            graph.replay()
        else:
            for i in range(steps):
                step(i)
        g1.record(stream)
    torch.cuda.synchronize()
    total_ms = g0.elapsed_time(g1)

    # The dominant kernel's own duration, from a HIP event pair bound to its
    # dispatch on this stream.  A fused step is one kernel: the steps run again,
    # each with its events.  Otherwise the step is the activation kernels then
    # the GEMM, and a start event bound to the GEMM would also take in the gap
    # after the kernel before it; the GEMM then runs back to back on the
    # activations of the last step (the same kernel on the same inputs).
    fam = kernel_family(M, K, args.variant, N)
    n_kt = min(steps, 512)
    evs = [(hip.event(), hip.event()) for _ in range(n_kt)]
    mm_prof = pkg.llmint8_matmul_fp8_profiled if fp8 else pkg.llmint8_matmul_profiled
    # The product's own workspace, as llmint8_matmul takes it: split-K partial
    # tiles and the weight codes at the outlier columns past the first 16,
    # with a small kernel ahead of the GEMM that zeroes the split counters and
    # gathers the codes.
    mm_ws = pkg.matmul_workspace(M, N, K, dev)

    def gemm_only(i, ev):
        CB, SCB = weights[i % n_copies]
        mm_prof(wl.dtype, M, N, K, q.CA.data_ptr(), q.SCA.data_ptr(), q.idx.data_ptr(),
                q.n_out.data_ptr(), q.XO.data_ptr(), CB.data_ptr(), SCB.data_ptr(),
                None if bias is None else bias.data_ptr(), Y.data_ptr(), None,
                mm_ws[0].data_ptr(), mm_ws[1], s_ptr, ev[0], ev[1])

    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        for i in range(n_kt):
            if fam in ("decode", "fused"):
                step(i, evs[i])
            else:
                gemm_only(i, evs[i])
    torch.cuda.synchronize()
    kern_ms = [hip.elapsed_ms(a, b) for a, b in evs]

    ms_per_step = total_ms / steps
    tops = 2.0 * M * N * K / (ms_per_step * 1e-3) / 1e12
    k_ms = float(np.mean(kern_ms))
    alg_bytes = algorithmic_bytes(fam, M, N, K, n_out, bias is not None)
    if fam != "tiled":
        achieved = alg_bytes / (k_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4)}
    else:
        peak = FP8_PEAK_TFLOPS if fp8 else INT8_PEAK_TOPS
        achieved = 2.0 * M * N * K / (k_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak,
                "unit": "TFLOP/s" if fp8 else "TOP/s", "frac": round(achieved / peak, 4)}
    ceiling = measured_ceiling(torch, pkg, dev, roof["bound"], fp8)
    ceiling["frac"] = round(roof["achieved"] / ceiling["value"], 4)
    roof["measured_peak"] = ceiling
    roof["traffic"] = load_traffic(args.config, fam, args.variant, args.threshold)
    roof["kernel"] = KERNEL_NAMES[fam]
    roof["kernel_ms"] = round(k_ms, 5)
    roof["algorithmic_bytes"] = alg_bytes
    roof["ops"] = 2 * M * N * K

    result = {
        "metric": METRIC, "value": round(tops, 3), "unit": "TOPS", "n_gpus": 1,
        "steps": steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8_e4m3" if fp8 else "int8",
        "data": "synthetic",
        "config": {"workload": f"{args.config}{' (FP8 E4M3 variant)' if fp8 else ''}: "
                               f"X {synth.DTYPE_NAMES[wl.dtype]} [{M}x{K}], "
                               f"W [{N}x{K}], threshold {wl.threshold}, {n_out} outlier columns"
                               + (", bias" if bias is not None else ""),
                   "M": M, "N": N, "K": K, "io_dtype": synth.DTYPE_NAMES[wl.dtype],
                   "outlier_cols": n_out, "threshold": wl.threshold, "variant": args.variant,
                   "weight_copies_rotated": n_copies, "graph": graph is not None},
        "roofline": roof,
        "weight_quant_once": {"ms": round(wq_ms, 4), "GB/s": round(wq_bytes / wq_ms / 1e6, 1),
                              "frac_hbm": round(wq_bytes / wq_ms / 1e6 / HBM_PEAK_GBS, 4)},
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"], result["cpu_baseline_1core"] = cpu_baseline(wl, variant=args.variant)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
