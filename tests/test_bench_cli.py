"""bench.py's command line on the CPU: one GPU only, and the arguments the profiles use."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120, cwd=ROOT)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = _bench("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_help_lists_the_figures_options():
    r = _bench("--help")
    assert r.returncode == 0
    for opt in ("--decode-rows", "--decode-only", "--paged-rows", "--pool", "--grouped",
                "--no-cpu-baseline", "--calib-copy-mib"):
        assert opt in r.stdout, opt
