"""Build libdcp.so (HIP, gfx950) in-tree with hipcc.

Each translation unit is compiled to an object in parallel, then linked into
``decode_attention_sequence_amd/libdcp.so``. Usage: ``python -m
decode_attention_sequence_amd.build [-v] [--host-sanitizers]``.

``--host-sanitizers`` builds a second copy, ``_build/sanitize/libdcp_host_sanitized.so``,
whose host code runs under AddressSanitizer and UndefinedBehaviorSanitizer
(device code unchanged). It needs the sanitizer runtime preloaded into the
process that loads it; the CPU tests use it to drive the C ABI's argument checks.
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


# Host-only sanitizers: each -fsanitize= goes to the host compilation alone.
HOST_SANITIZE_FLAGS = [
    "-Xarch_host", "-g",
    "-Xarch_host", "-fsanitize=address",
    "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=all",
    "-Xarch_host", "-fno-omit-frame-pointer",
]
SANITIZED_LIB = BUILD_DIR / "sanitize" / "libdcp_host_sanitized.so"


def _compile(src: str, verbose: bool, extra, out_dir: Path = BUILD_DIR) -> Path:
    obj = out_dir / (Path(src).stem + ".o")
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


def _link(objs, lib: Path) -> Path:
    tmp = lib.with_suffix(".so.tmp")
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", str(tmp), *map(str, objs)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, lib)
    return lib


def build(verbose: bool = False, extra_flags=()) -> Path:
    BUILD_DIR.mkdir(exist_ok=True)
    with ThreadPoolExecutor(min(len(SOURCES), 8)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, list(extra_flags)), SOURCES))
    _link(objs, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


def build_host_sanitized(verbose: bool = False) -> Path:
    """The library with AddressSanitizer and UndefinedBehaviorSanitizer on its
    host code, rebuilt when a source or header is newer than it. The sanitizer
    symbols stay undefined in the library: load it only into a process that
    has the runtime (libclang_rt.asan) preloaded."""
    out = SANITIZED_LIB.parent
    out.mkdir(parents=True, exist_ok=True)
    inputs = [*CSRC.iterdir(), *INCLUDE.iterdir(), Path(__file__)]
    if SANITIZED_LIB.exists() and all(p.stat().st_mtime <= SANITIZED_LIB.stat().st_mtime for p in inputs):
        return SANITIZED_LIB
    with ThreadPoolExecutor(min(len(SOURCES), 8)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, HOST_SANITIZE_FLAGS, out), SOURCES))
    _link(objs, SANITIZED_LIB)
    if verbose:
        print(f"built {SANITIZED_LIB}")
    return SANITIZED_LIB


if __name__ == "__main__":
    if "--host-sanitizers" in sys.argv:
        build_host_sanitized(verbose="-v" in sys.argv)
    else:
        build(verbose="-v" in sys.argv)
