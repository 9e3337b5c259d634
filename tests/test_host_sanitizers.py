"""The library's host code -- the partition layout and the threaded host AdamW
of the offload path -- built with AddressSanitizer + UndefinedBehaviorSanitizer
and, separately, ThreadSanitizer (host code only: no GPU pass), and driven by
tests/host_sanitizer_driver.cpp: 300 random layouts with every rank's fragment
list, and host AdamW at ragged sizes, offsets and thread counts from four
threads at once.  Any sanitizer report fails the test."""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "zero_sharded_optimizer_zr_amd", "csrc")
SOURCES = [os.path.join(CSRC, "layout.cpp"), os.path.join(CSRC, "offload.cpp"),
           os.path.join(ROOT, "tests", "host_sanitizer_driver.cpp")]

pytestmark = pytest.mark.skipif(shutil.which("hipcc") is None, reason="hipcc not available")


def build(tmp, sanitize):
    flags = ["--offload-arch=gfx950", "--offload-host-only", "-O1", "-g", "-std=c++17", "-fno-omit-frame-pointer",
             "-ffp-contract=off", f"-I{ROOT}/include", f"-I{CSRC}"]
    san = [x for s in sanitize for x in ("-Xarch_host", f"-fsanitize={s}")]
    objs = [os.path.join(tmp, os.path.basename(src).replace(".", "_") + ".o") for src in SOURCES]
    with ThreadPoolExecutor(3) as pool:
        rs = list(pool.map(lambda so: subprocess.run(["hipcc", *flags, *san, "-c", so[0], "-o", so[1]],
                                                     capture_output=True, text=True), zip(SOURCES, objs)))
    for r in rs:
        assert r.returncode == 0, r.stderr[-2000:]
    exe = os.path.join(tmp, "driver_" + "_".join(sanitize))
    r = subprocess.run(["hipcc", *san, *objs, "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return exe


@pytest.mark.parametrize("sanitize", [("address", "undefined"), ("thread",)], ids=["asan_ubsan", "tsan"])
def test_host_code_is_clean_under_sanitizers(tmp_path, sanitize):
    exe = build(str(tmp_path), sanitize)
    env = {**os.environ, "ASAN_OPTIONS": "detect_leaks=1:halt_on_error=1",
           "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1", "TSAN_OPTIONS": "halt_on_error=1"}
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=900)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "Sanitizer" not in r.stderr and r.stdout.startswith("ok:"), r.stderr[-4000:]
