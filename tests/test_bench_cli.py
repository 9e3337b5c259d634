"""bench.py's command line on the CPU: it measures one GPU only, so any other
--gpus value exits with status 2 and says why, before touching a device."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    for n in ("2", "8"):
        r = run("--gpus", n)
        assert r.returncode == 2
        assert "one GPU only" in r.stderr and r.stdout == ""


def test_help_lists_the_contract_flags():
    r = run("--help")
    assert r.returncode == 0
    for flag in ("--gpus", "--steps", "--warmup", "--workload"):
        assert flag in r.stdout
