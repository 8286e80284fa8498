"""Build libgqa_decode.so in-tree with hipcc for gfx950.

    python -m gqa_kv_cache_decode_amd.build          # or build_library()

Every HIP source is compiled to an object under ``_build/`` and linked into
``gqa_kv_cache_decode_amd/libgqa_decode.so``.  Always recompiles.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
INCLUDE = ROOT / "include"
BUILD = ROOT / "_build"
LIB = PKG / "libgqa_decode.so"
BENCH_LIB = PKG / "libgqa_bench.so"   # measurement helpers, not the decode ABI
ARCH = "gfx950"

SOURCES = ["abi.cpp", "append.hip", "partition_bf16.hip", "partition_fp8.hip",
           "noalloc.hip",
           "partition_f32.hip",
           "combine.hip", "schedule.hip"]
BENCH_SOURCES = ["bench_kernels.hip"]

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-fvisibility=hidden",
    "-Wall", "-Wno-unused-command-line-argument",
    f"-I{INCLUDE}", f"-I{CSRC}",
]
# Packed fp32 VALU ops stay off: the compiler must not form them by itself.
DEVICE_ONLY = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# The partition kernels take work-queue items with a single-lane atomic whose
# result is needed only after the current item: the wave-level atomic
# rewrite would wait for it at once (it combines the lanes' results).
PER_SOURCE = {s: ["-mllvm", "-amdgpu-atomic-optimizer-strategy=None"]
              for s in ("partition_bf16.hip", "partition_fp8.hip")}


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; ROCm is required to build")
    return path


def _compile(src: str) -> Path:
    obj = BUILD / (src + ".o")
    cmd = [hipcc(), *COMMON]
    if src.endswith(".hip"):
        cmd += DEVICE_ONLY
    cmd += PER_SOURCE.get(src, [])
    cmd += ["-c", str(CSRC / src), "-o", str(obj)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stdout}\n{res.stderr}")
    return obj


def _link(objs, lib: Path) -> None:
    tmp = lib.with_suffix(".so.tmp")
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC",
           *map(str, objs), "-o", str(tmp)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link of {lib.name} failed:\n{res.stdout}\n"
                           f"{res.stderr}")
    os.replace(tmp, lib)


def build_library(verbose: bool = False) -> Path:
    BUILD.mkdir(exist_ok=True)
    srcs = SOURCES + BENCH_SOURCES
    with cf.ThreadPoolExecutor(max_workers=min(len(srcs), 8)) as ex:
        objs = dict(zip(srcs, ex.map(_compile, srcs)))
    _link([objs[s] for s in SOURCES], LIB)
    _link([objs[s] for s in BENCH_SOURCES], BENCH_LIB)
    if verbose:
        print(f"built {LIB} and {BENCH_LIB}")
    return LIB


if __name__ == "__main__":
    build_library(verbose=True)
    sys.exit(0)
