"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The library is rebuilt with both sanitizers on its host code (device code
unchanged; `decode_attention_sequence_amd.build.build_host_sanitized`), and
tests/test_lib_abi.py runs against that build in a child Python process with
the sanitizer runtime preloaded. Every call there is an argument check, a
workspace-size query or a symbol lookup, so no GPU is needed. Any sanitizer
report fails the run.
"""
import os
import shutil
import subprocess
import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parent.parent
CLANG = Path("/opt/rocm/lib/llvm/bin/clang")


def _asan_runtime():
    if not CLANG.exists():
        return None
    out = subprocess.run([str(CLANG), "-print-file-name=libclang_rt.asan-x86_64.so"],
                         capture_output=True, text=True).stdout.strip()
    return out if os.path.isabs(out) and os.path.exists(out) else None


@pytest.mark.skipif(shutil.which("hipcc") is None and not Path("/opt/rocm/bin/hipcc").exists(),
                    reason="hipcc missing")
def test_abi_checks_under_host_sanitizers(tmp_path):
    from decode_attention_sequence_amd import build

    runtime = _asan_runtime()
    if runtime is None:
        pytest.skip("the clang AddressSanitizer runtime is not installed")
    lib = build.build_host_sanitized()
    logs = tmp_path / "reports"
    env = dict(os.environ,
               LD_PRELOAD=runtime,
               DCP_LIBRARY=str(lib),
               ASAN_OPTIONS=f"detect_leaks=0:alloc_dealloc_mismatch=0:halt_on_error=1:log_path={logs}",
               UBSAN_OPTIONS=f"halt_on_error=1:print_stacktrace=1:log_path={logs}")
    run = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                          str(ROOT / "tests" / "test_lib_abi.py")],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    reports = "".join(p.read_text() for p in tmp_path.glob("reports*"))
    assert run.returncode == 0 and not reports, (run.stdout[-4000:] + run.stderr[-2000:] + reports[:4000])
    assert " passed" in run.stdout
