"""Build libdcp.so (HIP, gfx950) in-tree with hipcc.

Each translation unit is compiled to an object in parallel, then linked into
``decode_attention_sequence_amd/libdcp.so``. Usage: ``python -m
decode_attention_sequence_amd.build [-v]``.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
INCLUDE = ROOT / "include"
BUILD_DIR = ROOT / "_build"
LIB = PKG / "libdcp.so"
SOURCES = ["api.hip", "plan_merge.hip", "mla.hip", "gqa.hip", "append.hip"]
ARCH = "gfx950"

# Packed-fp32 VALU ops are switched off for all device code.
HIP_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the HIP toolchain is required to build libdcp")
    return path


def _compile(src: str, verbose: bool, extra) -> Path:
    obj = BUILD_DIR / (Path(src).stem + ".o")
    cmd = [hipcc(), *HIP_FLAGS, *extra, "-c", str(CSRC / src), "-o", str(obj)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    # The host pass warns that it does not know the packed-fp32 target feature.
    err = "\n".join(line for line in res.stderr.splitlines()
                    if "is not a recognized feature for this target" not in line)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    return obj


def build(verbose: bool = False, extra_flags=()) -> Path:
    BUILD_DIR.mkdir(exist_ok=True)
    with ThreadPoolExecutor(min(len(SOURCES), 8)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, list(extra_flags)), SOURCES))
    tmp = LIB.with_suffix(".so.tmp")
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", str(tmp), *map(str, objs)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
