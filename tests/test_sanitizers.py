"""The oracle and the C ABI's host-side validation under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only).

Two drivers in tests/sanitize/ are built with the sanitizers and run as child
processes: oracle_driver.c runs every oracle function on small and edge-case
inputs; abi_driver.c calls every C-ABI entry point with arguments its
validation must refuse, and every size query over extreme shapes, so no call
reaches the GPU.  The library's other objects (the kernels' host stubs) are
linked uninstrumented.  A sanitizer finding aborts the child.
"""
import glob
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
SAN_ENV = dict(os.environ,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
ROCM = "/opt/rocm"


def run(cmd, **kw):
    p = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert p.returncode == 0, f"{' '.join(cmd)}\n{p.stdout}\n{p.stderr}"
    return p


def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_san")
    run(["gcc", "-O1", "-g", "-std=c11", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
         "-ffp-contract=off", "-fno-fast-math", "-Wall",
         os.path.join(ROOT, "oracle", "llmint8_oracle.c"), os.path.join(HERE, "oracle_driver.c"),
         "-o", exe, "-lm"])
    p = run([exe], env=SAN_ENV, timeout=300)
    assert "oracle driver: ok" in p.stdout
    assert "runtime error" not in p.stderr


@pytest.mark.skipif(not os.path.exists(f"{ROCM}/bin/hipcc"), reason="needs hipcc")
def test_abi_validation_under_asan_ubsan(tmp_path):
    from int8_quantized_matmul_row_amd import build as hipbuild
    objs = [o for o in glob.glob(os.path.join(ROOT, "_build", "*.o")) if not o.endswith("/api.o")]
    if not objs:
        hipbuild.build()
        objs = [o for o in glob.glob(os.path.join(ROOT, "_build", "*.o")) if not o.endswith("/api.o")]
    api_o = str(tmp_path / "api_san.o")
    # host-side instrumentation only: each -fsanitize= follows -Xarch_host
    run([f"{ROCM}/bin/hipcc", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
         "-Xarch_host", "-fno-sanitize-recover=all",
         "-I", os.path.join(ROOT, "include"),
         "-c", os.path.join(ROOT, "int8_quantized_matmul_row_amd", "csrc", "api.hip"), "-o", api_o])
    drv_o = str(tmp_path / "abi_driver.o")
    run([f"{ROCM}/llvm/bin/clang", "-O1", "-g", "-std=c11", "-fsanitize=address,undefined",
         "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
         "-I", f"{ROCM}/include", "-c", os.path.join(HERE, "abi_driver.c"), "-o", drv_o])
    exe = str(tmp_path / "abi_san")
    run([f"{ROCM}/llvm/bin/clang++", "-fsanitize=address,undefined", drv_o, api_o, *objs,
         f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib", "-o", exe])
    p = run([exe], env=SAN_ENV, timeout=300)
    assert "abi driver: ok" in p.stdout
    assert "runtime error" not in p.stderr
