"""Build the HIP library in-tree: ``hipcc --offload-arch=gfx950`` for every source, one shared object.

    python -m moe_expert_layer_amd.build          # or: from moe_expert_layer_amd.build import build

``build()`` also builds the probe library (the same sources with ``MOE_PHASE_PROBE``: the bf16
GEMMs add per-task cycle stamps and export ``moe_probe_phases``), which ``bench.py --phase-probe``
loads instead of the product library.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_NAME = "libmoe_expert_layer.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
PROBE_LIB_PATH = os.path.join(HERE, "libmoe_expert_layer_probe.so")

SOURCES = ["api.cpp", "route.hip", "permute.hip", "gemm_f32.hip", "gemm_bf16.hip", "gemm_mx.hip",
           "router.hip", "gemm_bwd.hip"]
HEADERS = ["common.h", "internal.h", "gemm_common.h"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    # no packed fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def _compile(src: str, out_dir: str, defines: tuple) -> str:
    obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
    flags = [*FLAGS, *(f"-D{d}" for d in defines)]
    cmd = [HIPCC, *flags, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd = [HIPCC, *flags, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def _build_one(lib_path: str, out_dir: str, defines: tuple, verbose: bool) -> str:
    os.makedirs(out_dir, exist_ok=True)
    workers = max(1, min(len(SOURCES), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4))))
    with ThreadPoolExecutor(workers) as ex:
        objs = list(ex.map(lambda src: _compile(src, out_dir, defines), SOURCES))
    tmp = lib_path + ".tmp"
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib_path)
    if verbose:
        print(f"built {lib_path}")
    return lib_path


def build(verbose: bool = True, probe: bool = True) -> str:
    """Compile every source and link the shared library, then (probe) the probe library (always
    rebuilds).  Returns the product library's path."""
    _build_one(LIB_PATH, BUILD_DIR, (), verbose)
    if probe:
        _build_one(PROBE_LIB_PATH, BUILD_DIR + "_probe", ("MOE_PHASE_PROBE",), verbose)
    return LIB_PATH


if __name__ == "__main__":
    build()
    sys.exit(0)
