"""Compile the sources of the library into ``libpagedkv.so``: HIP for gfx950, host C++.

``python -m paged_kv_cache_294_amd.build`` (or :func:`build`) runs hipcc once per source
file, in parallel, then links the shared library next to this file. It always rebuilds.
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_NAME = "libpagedkv.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
ARCH = "gfx950"

SOURCES = ["pa_api.hip", "kv_append.hip", "pa_decode.hip", "pa_prefill.hip", "pa_gather.hip",
           "pa_blocks.hip", "block_manager.cpp"]

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fvisibility=hidden",
    "-Wall",
    "-Wno-unused-result",
    # no packed-fp32 instructions in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix-core results in ordinary VGPRs rather than accumulation registers: the fp16
    # grouped-query decode kernel then needs 154 registers instead of 154 + 32 (three
    # waves per SIMD instead of two); its FP8 variant, which keeps the loaded codes packed
    # and two blocks in flight, needs 138 (129 in shared-prefix decode; three waves)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-Wall"]


def cxx() -> str:
    path = shutil.which("g++") or shutil.which("c++")
    if path is None:
        raise RuntimeError("no host C++ compiler found")
    return path


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the ROCm toolchain is needed to build the library")
    return path


def _compile(src: str, extra) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    if src.endswith(".cpp"):  # host-only code
        cmd = [cxx(), *HOST_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    else:
        cmd = [hipcc(), *HIPCC_FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compiler failed on {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False, extra_flags=()) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, list(extra_flags)), SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH}")
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True, extra_flags=sys.argv[1:])
