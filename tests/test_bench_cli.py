"""bench.py's command line, checked without touching a GPU: a request for more
than one GPU is refused with a message, and the help lists the options."""
import subprocess
import sys
from pathlib import Path

ROOT = Path(__file__).resolve().parent.parent


def _run(*args):
    return subprocess.run([sys.executable, str(ROOT / "bench.py"), *args], capture_output=True,
                          text=True, timeout=300, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_help_lists_the_workloads_and_q_len():
    r = _run("--help")
    assert r.returncode == 0
    assert "mla_bf16_b64_bimodal" in r.stdout and "--q-len" in r.stdout
