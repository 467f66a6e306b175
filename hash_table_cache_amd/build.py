"""Builds the HIP library ``_lib/libhkv.so`` for gfx950 with hipcc.

Run as ``python -m hash_table_cache_amd.build``. Cross-compiles without a GPU.
"""

from __future__ import annotations

import os
import pathlib
import subprocess
import sys

PKG = pathlib.Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
INCLUDE = ROOT / "include"
BUILD_DIR = PKG / "_build"
LIB_PATH = PKG / "_lib" / "libhkv.so"

SOURCES = [CSRC / "hkv_kernels.hip", CSRC / "hkv_runtime.cpp"]
# multi-threaded driver of the mixed reader/updater/inserter benchmark, a
# library of its own on top of the C ABI
MIXED_SOURCE = CSRC / "hkv_mixed_driver.cpp"
MIXED_LIB_PATH = PKG / "_lib" / "libhkv_mixed.so"
# access-pattern ceiling of find (a stand-alone benchmark program)
PATTERN_SOURCE = CSRC / "hkv_pattern_ceiling.hip"
PATTERN_EXE = PKG / "_lib" / "hkv_pattern_ceiling"
ARCH = "gfx950"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return str(pathlib.Path(rocm) / "bin" / "hipcc")


def compile_flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-fvisibility=hidden",
        # packed fp32 instructions stay off (no float arithmetic here anyway)
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall",
        "-I", str(INCLUDE),
        "-I", str(CSRC),
    ]


def build(verbose: bool = False) -> pathlib.Path:
    BUILD_DIR.mkdir(parents=True, exist_ok=True)
    LIB_PATH.parent.mkdir(parents=True, exist_ok=True)
    objs = []
    for src in SOURCES:
        obj = BUILD_DIR / (src.name + ".o")
        lang = ["-x", "hip"] if src.suffix == ".hip" else []
        cmd = [hipcc(), *compile_flags(), *lang, "-c", str(src), "-o", str(obj)]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True, stderr=None if verbose else subprocess.PIPE)
        objs.append(obj)
    tmp = LIB_PATH.with_suffix(".so.tmp")
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", str(tmp), *map(str, objs)]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    tmp.replace(LIB_PATH)
    obj = BUILD_DIR / (MIXED_SOURCE.name + ".o")
    cmd = [hipcc(), *compile_flags(), "-c", str(MIXED_SOURCE), "-o", str(obj)]
    subprocess.run(cmd, check=True, stderr=None if verbose else subprocess.PIPE)
    tmp = MIXED_LIB_PATH.with_suffix(".so.tmp")
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", str(tmp), str(obj),
           f"-L{LIB_PATH.parent}", "-lhkv", "-Wl,-rpath,$ORIGIN", "-pthread"]
    subprocess.run(cmd, check=True)
    tmp.replace(MIXED_LIB_PATH)
    tmp = PATTERN_EXE.with_suffix(".tmp")
    cmd = [hipcc(), *[f for f in compile_flags() if f != "-fvisibility=hidden"], "-x", "hip", str(PATTERN_SOURCE),
           "-o", str(tmp)]
    subprocess.run(cmd, check=True, stderr=None if verbose else subprocess.PIPE)
    tmp.replace(PATTERN_EXE)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
