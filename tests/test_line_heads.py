"""The vector-body heads of the streaming kernels (host code): built host-only
and run over every address phase (tests/host_line_heads.cpp)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "zero_sharded_optimizer_zr_amd", "csrc")

pytestmark = pytest.mark.skipif(shutil.which("hipcc") is None, reason="hipcc not available")


def test_line_heads(tmp_path):
    exe = str(tmp_path / "line_heads")
    r = subprocess.run(["hipcc", "--offload-arch=gfx950", "--offload-host-only", "-O1", "-std=c++17",
                        f"-I{ROOT}/include", f"-I{CSRC}", os.path.join(ROOT, "tests", "host_line_heads.cpp"),
                        "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and r.stdout.startswith("ok:"), (r.stdout + r.stderr)[-2000:]
