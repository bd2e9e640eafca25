"""Ahead-of-time build of libpkv.so for gfx950 (hipcc, in-tree).

Every source is compiled by hipcc for a single offload arch and linked into
one shared library next to this file. Packed-fp32 instructions are disabled
(`-packed-fp32-ops`), so the compiler never emits v_pk_{add,mul,fma}_f32.
"""

from __future__ import annotations

import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(HERE, "libpkv.so")
SOURCES = ["api.cpp", "planner.cpp", "decode.hip", "merge.hip", "prefill.hip", "append.hip", "pod.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def common_flags() -> list[str]:
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-I", INCLUDE, "-I", CSRC,
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-function", "-Wno-unused-variable"]


# The debug variant: the prefill kernels fill their LDS tile buffers with NaN
# before each item (PKV_DEBUG_LDS_POISON), for the tests of the counted waits.
DEBUG_LIB_PATH = os.path.join(HERE, "libpkv_debug.so")
DEBUG_DEFINES = ["-DPKV_DEBUG_LDS_POISON"]


def _compile(job) -> str:
    src, build_dir, defines = job
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [hipcc()] + common_flags() + defines + ["-x", "hip", "-c", os.path.join(CSRC, src),
                                                  "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stdout}\n{res.stderr}")
    return obj


def _link(objs, path):
    tmp = path + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, path)


def build(verbose: bool = False) -> str:
    """Compile every source and link libpkv.so (and its debug variant
    libpkv_debug.so); returns the library path."""
    debug_dir = os.path.join(BUILD_DIR, "debug")
    os.makedirs(debug_dir, exist_ok=True)
    jobs = [(s, BUILD_DIR, []) for s in SOURCES] + [(s, debug_dir, DEBUG_DEFINES) for s in SOURCES]
    with ThreadPoolExecutor(max_workers=8) as pool:
        objs = list(pool.map(_compile, jobs))
    _link(objs[:len(SOURCES)], LIB_PATH)
    _link(objs[len(SOURCES):], DEBUG_LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH} and {DEBUG_LIB_PATH}")
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
