"""Build libllmint8.so (HIP, gfx950) in-tree with hipcc.

    python -m int8_quantized_matmul_row_amd.build [--asm]

Each csrc/*.hip is compiled to an object under _build/ (in parallel), then
linked into int8_quantized_matmul_row_amd/libllmint8.so.  --asm also keeps the
gfx950 assembly (_build/*.s) for register and instruction checks.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIBRARY = os.path.join(PKG, "libllmint8.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
    # packed fp32 instructions stay off: ordinary float code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def _run(cmd):
    p = subprocess.run(cmd, capture_output=True, text=True)
    noise = ("packed-fp32-ops", "warning: unknown target feature", "1 warning generated")
    err = "\n".join(l for l in p.stderr.splitlines() if not any(n in l for n in noise)
                    and l.strip())
    if p.returncode != 0:
        raise RuntimeError(f"command failed: {' '.join(cmd)}\n{p.stderr}")
    return err


def build(asm: bool = False, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objs = []
    cmds = []
    for src in sources:
        obj = os.path.join(BUILD, os.path.basename(src)[:-4] + ".o")
        objs.append(obj)
        cmds.append([HIPCC, *HIP_FLAGS, "-c", src, "-o", obj])
        if asm:
            s = os.path.join(BUILD, os.path.basename(src)[:-4] + ".s")
            cmds.append([HIPCC, *HIP_FLAGS, "--cuda-device-only", "-S", src, "-o", s])
    with cf.ThreadPoolExecutor(max_workers=min(8, len(cmds))) as ex:
        for msg in ex.map(_run, cmds):
            if msg and verbose:
                print(msg, file=sys.stderr)
    tmp = LIBRARY + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    print(build(asm="--asm" in sys.argv, verbose=True))
