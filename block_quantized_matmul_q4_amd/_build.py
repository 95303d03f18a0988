"""Ahead-of-time build of ``libqmm.so`` for gfx950 with hipcc.

Every translation unit is compiled in-tree (the .so travels with the source
tree) with packed-FP32 instruction selection disabled.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import pathlib
import subprocess
import sys

HERE = pathlib.Path(__file__).resolve().parent
CSRC = HERE / "csrc"
INCLUDE = HERE.parent / "include"
LIBRARY = HERE / "libqmm.so"
BUILD_DIR = HERE.parent / "_build"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-Wall", "-Werror", "-Wno-unused-function",
    # never let the compiler form v_pk_{add,mul,fma}_f32
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # private arrays stay in registers; never silently moved into LDS
    "-mllvm", "-disable-promote-alloca-to-lds",
    f"-I{INCLUDE}",
]


def sources():
    return sorted(CSRC.glob("*.hip"))


def _compile(src: pathlib.Path) -> pathlib.Path:
    obj = BUILD_DIR / (src.stem + ".o")
    cmd = [HIPCC, *FLAGS, "-c", str(src), "-o", str(obj)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src.name}:\n{res.stderr}")
    return obj


def build(verbose: bool = False) -> pathlib.Path:
    BUILD_DIR.mkdir(exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, sources()))
    tmp = LIBRARY.with_name(LIBRARY.name + ".tmp")
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", str(tmp),
           *map(str, objs)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    tmp.replace(LIBRARY)
    if verbose:
        print(LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
