"""Build libggrms.so (and the benchmark's helper library) in-tree for gfx950.

Each HIP translation unit compiles on its own hipcc process (in parallel),
then hipcc links the shared library next to this file.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libggrms.so")
BENCH_LIB = os.path.join(PKG, "libggrms_bench.so")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed-FP32 instructions are kept out of the generated code; the feature
# flag only means something to the device pass (the host pass warns).
HIP_FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", INCLUDE, "-I", CSRC]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-I", INCLUDE, "-I", CSRC]

LIB_HIP = ["ggrms_api.hip", "table_f32.hip", "table_f16.hip", "table_bf16.hip",
           "table_f32_nbg.hip", "table_f16_nbg.hip", "table_bf16_nbg.hip"]
LIB_CXX = ["plan.cpp"]
BENCH_HIP = ["bench_aux.hip"]
# the epilogue called from a producer kernel (an example, not part of the ABI)
EXAMPLE_HIP = ["example_producer.hip"]
EXAMPLE_LIB = os.path.join(PKG, "libggrms_example.so")


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return r


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    path = os.path.join(CSRC, src)
    # the product library exports its C ABI only (GGRMS_API in ggrms.h)
    vis = ["-fvisibility=hidden"] if src in LIB_HIP + LIB_CXX else []
    if src.endswith(".hip"):
        _run([HIPCC, *HIP_FLAGS, *vis, "-c", path, "-o", obj])
    else:
        _run(["g++", *CXX_FLAGS, *vis, "-c", path, "-o", obj])
    return obj


def _link(objs, out, libs=()):
    tmp = out + f".tmp{os.getpid()}"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs, *libs])
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    """Compile every HIP source for gfx950 and link libggrms.so and libggrms_bench.so."""
    if shutil.which(HIPCC) is None and not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(BUILD, exist_ok=True)
    srcs = LIB_HIP + LIB_CXX + BENCH_HIP + EXAMPLE_HIP
    with cf.ThreadPoolExecutor(min(8, len(srcs))) as ex:
        objs = dict(zip(srcs, ex.map(_compile, srcs)))
    _link([objs[s] for s in LIB_HIP + LIB_CXX], LIB,
          [f"-Wl,--version-script={os.path.join(CSRC, 'libggrms.map')}"])
    # the benchmark helpers call the product library itself (found next to them)
    _link([objs[s] for s in BENCH_HIP], BENCH_LIB,
          ["-L", PKG, "-l:libggrms.so", "-Wl,-rpath,$ORIGIN"])
    _link([objs[s] for s in EXAMPLE_HIP], EXAMPLE_LIB)
    if verbose:
        print(f"built {LIB}, {BENCH_LIB} and {EXAMPLE_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
