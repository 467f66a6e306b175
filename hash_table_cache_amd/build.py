"""Builds the HIP library ``_lib/libhkv.so`` for gfx950 with hipcc, and the
multi-threaded mixed-workload driver ``_lib/libhkv_mixed.so`` on top of it.

Run as ``python -m hash_table_cache_amd.build``. Cross-compiles without a GPU.
The objects compile in parallel.
"""

from __future__ import annotations

import concurrent.futures
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


def _run(cmd: list[str], verbose: bool) -> None:
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stderr=subprocess.PIPE, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stderr)
        raise subprocess.CalledProcessError(r.returncode, cmd)
    if verbose and r.stderr:
        sys.stderr.write(r.stderr)


def _compile(src: pathlib.Path, verbose: bool) -> pathlib.Path:
    obj = BUILD_DIR / (src.name + ".o")
    lang = ["-x", "hip"] if src.suffix == ".hip" else []
    _run([hipcc(), *compile_flags(), *lang, "-c", str(src), "-o", str(obj)], verbose)
    return obj


def build(verbose: bool = False) -> pathlib.Path:
    BUILD_DIR.mkdir(parents=True, exist_ok=True)
    LIB_PATH.parent.mkdir(parents=True, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=3) as pool:
        futs = [pool.submit(_compile, src, verbose) for src in (*SOURCES, MIXED_SOURCE)]
        objs = [f.result() for f in futs]
    tmp = LIB_PATH.with_suffix(".so.tmp")
    _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", str(tmp), *map(str, objs[:2])], verbose)
    tmp.replace(LIB_PATH)
    tmp = MIXED_LIB_PATH.with_suffix(".so.tmp")
    _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", str(tmp), str(objs[2]),
          f"-L{LIB_PATH.parent}", "-lhkv", "-Wl,-rpath,$ORIGIN", "-pthread"], verbose)
    tmp.replace(MIXED_LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
