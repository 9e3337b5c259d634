"""bench.py's output line on the tiny MLP shard: one JSON object on the last
line of stdout carrying the fields the measurement contract names (metric,
value, unit, step counts, timing, dtype, workload config, the roofline object
of the AdamW kernel and the oracle's CPU baseline), with values that agree with
one another.  bench.py runs as a child process, as a user would run it."""
import json
import os
import subprocess
import sys

import pytest

from gpu_util import device, say

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_line_on_the_tiny_shard():
    device()
    cmd = [sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "tiny_mlp_nd4_r0", "--steps", "3",
           "--warmup", "1", "--no-extra-paths", "--cpu-seconds", "0.5"]
    say("bench.py", " ".join(cmd[2:]))
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=110, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    line = json.loads(r.stdout.strip().splitlines()[-1])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in line, key
    assert line["n_gpus"] == 1 and line["steps"] == 3 and line["warmup"] == 1
    assert line["higher_is_better"] is True and line["vs_baseline"] is None
    assert line["config"]["workload"] == "tiny_mlp_nd4_r0"
    assert line["value"] > 0 and line["ms_per_step"] > 0
    # value is shard elements per second of the whole step
    assert line["value"] == pytest.approx(262_144 / (line["ms_per_step"] * 1e-3), rel=1e-2)  # ms rounded to 1e-4
    roof = line["roofline"]
    assert roof["bound"] == "hbm" and roof["unit"] == "GB/s" and roof["peak"] == 8000.0
    assert roof["frac"] == pytest.approx(roof["achieved"] / roof["peak"], abs=1e-3)
    assert roof["traffic"] is None          # counters were taken on the 7e9 shard only
    pat = roof["pattern_ceiling"]           # the AdamW access pattern without arithmetic, same buffers
    assert pat["ms_avg"] > 0 and pat["frac"] == pytest.approx(pat["GBps"] / roof["peak"], abs=1e-3)
    assert pat["adamw_over_pattern"] == pytest.approx(pat["ms_avg"] / roof["algorithmic_bytes_per_launch"]
                                                      * roof["achieved"] * 1e6, rel=1e-2)
    cpu = line["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["value"] > 0 and cpu["cores"] >= 1 and cpu["sample"]
