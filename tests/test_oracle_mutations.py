"""Pin strength: plant one plausible mistake at a time in a scratch copy of the
oracle (CPU only) and check that the oracle's pin tests then fail."""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

C = "oracle/zr_oracle.c"
PY = "oracle/__init__.py"
MUTATIONS = [
    ("dropped weight decay", C, "th = th * decay;", "th = th;"),
    ("wrong update sign", C, "th = th - lr * m_hat", "th = th + lr * m_hat"),
    ("eps inside the root", C, "(sqrt(v_hat) + eps)", "sqrt(v_hat + eps)"),
    ("no first-moment bias correction", C, "double m_hat = m / bias1;", "double m_hat = m;"),
    ("wrong second-moment correction", C, "double v_hat = v / bias2;", "double v_hat = v / bias1;"),
    ("g instead of g^2", C, "(1.0 - beta2) * g * g", "(1.0 - beta2) * g"),
    ("beta1 for 1 - beta1", C, "m = beta1 * m + (1.0 - beta1) * g;", "m = beta1 * m + beta1 * g;"),
    ("grad_scale ignored", C, "double g = (double)bf16_to_f32(grad[i]) * grad_scale;",
     "double g = (double)bf16_to_f32(grad[i]);"),
    ("mean over n + 1", C, "float mean = sum / (float)n;", "float mean = sum / (float)(n + 1);"),
    ("last contribution dropped", C, "for (int32_t k = 1; k < n; ++k)", "for (int32_t k = 1; k < n - 1; ++k)"),
    ("ties always up", C, "(lower == 0x8000u && (upper & 1u))", "(lower == 0x8000u)"),
    ("bf16 copy off by one bit", C, "param_out[i] = f32_to_bf16(master[i]);",
     "param_out[i] = (uint16_t)(f32_to_bf16(master[i]) ^ 1);"),
    ("threshold inclusive", PY, "self.persistent = [x < self.threshold", "self.persistent = [x <= self.threshold"),
    ("padding always added", PY, "self.psi_pad = -(-self.psi_part // self.n_d) * self.n_d",
     "self.psi_pad = (self.psi_part // self.n_d) * self.n_d + self.n_d"),
    ("stage-2 ledger uses 12", PY, "return 2 * self.psi + 14 * owned", "return 2 * self.psi + 12 * owned"),
    ("stage-1 closed form uses 14", PY, "return 4 * psi + 12 * psi / n_d", "return 4 * psi + 14 * psi / n_d"),
    ("fragment one too long", PY, "out.append((t, lo - self.offset[t], lo, hi - lo))",
     "out.append((t, lo - self.offset[t], lo, hi - lo + (1 if hi < end else 0)))"),
    ("fp16 ties always up", C, "if (dropped > 0x1000u || (dropped == 0x1000u && (man & 1u)))",
     "if (dropped >= 0x1000u)"),
    ("fp16 subnormal threshold", C, "if (a < 6.103515625e-05f) {", "if (a < 3.0517578125e-05f) {"),
    ("loss scale not divided out", C, "double g = (double)f16_to_f32(grad[i]) * unscale * grad_scale;",
     "double g = (double)f16_to_f32(grad[i]) * grad_scale;"),
    ("found-inf misses inf", C, "if ((x[i] & 0x7c00u) == 0x7c00u)", "if ((x[i] & 0x7e00u) == 0x7e00u)"),
    ("fp16 mean over n - 1", C, "out[i] = f32_to_f16(sum / (float)n);", "out[i] = f32_to_f16(sum / (float)(n > 1 ? n - 1 : 1));"),
    ("loss-scale window off by one", PY, "if self.good_steps == self.window:",
     "if self.good_steps == self.window - 1:"),
    ("overflowing step not skipped", PY, "    if not inf:\n        adamw_f16(", "    if True:\n        adamw_f16("),
    ("backoff ignores the floor", PY, "self.scale = max(self.scale / self.factor, self.min_scale)",
     "self.scale = self.scale / self.factor"),
    ("int8 ties away from zero", C, "float r = rintf(bf16_to_f32(src[i]) / s);",
     "float r = roundf(bf16_to_f32(src[i]) / s);"),
    ("int8 scale over 128", C, "float s = amax / 127.0f;", "float s = amax / 128.0f;"),
    ("int8 absmax without abs", C, "float a = fabsf(bf16_to_f32(src[i]));", "float a = bf16_to_f32(src[i]);"),
    ("int8 dequant wrong block", C, "float x = (float)q[i] * scales[i / block];",
     "float x = (float)q[i] * scales[(i + 1) / block < (numel + block - 1) / block ? (i + 1) / block : i / block];"),
    ("gathered blocks not restarted per shard", PY, "return r * per_rank + (i - r * S) // block",
     "return i // block"),
    ("sub-range scales not offset", PY, "x = q[: end - begin].astype(np.float32) * scales[g - g[0]]",
     "x = q[: end - begin].astype(np.float32) * scales[g - g[0] + (1 if begin > 0 else 0)]"),
    ("int4 nibbles swapped", C, "q4[i / 2] |= (i % 2) ? (uint8_t)(nibble << 4) : nibble;",
     "q4[i / 2] |= (i % 2) ? nibble : (uint8_t)(nibble << 4);"),
    ("int4 scale over 8", C, "float s = amax / 7.0f;", "float s = amax / 8.0f;"),
    ("int4 clamp at 6", C, "if (r > 7.0f)\n                    r = 7.0f;", "if (r > 6.0f)\n                    r = 6.0f;"),
    ("int4 codes read unsigned", C, "int code = nibble >= 8 ? nibble - 16 : nibble;", "int code = nibble;"),
    ("int4 gathered bytes not restarted per shard", PY, "return r * (-(-S // 2)) + (i - r * S) // 2",
     "return i // 2"),
    ("unpack reversed", PY, "arr[toff - first: toff - first + n] = flat[foff - begin: foff - begin + n]",
     "arr[toff - first: toff - first + n] = flat[foff - begin: foff - begin + n][::-1]"),
]

PIN_TESTS = ["tests/test_oracle_numerics.py", "tests/test_oracle_layout.py", "tests/test_oracle_ledger.py",
             "tests/test_oracle_fp16.py", "tests/test_oracle_int8.py", "tests/test_oracle_int4.py"]


def _plant_and_run(root, what, path, old, new):
    """Copies the oracle and its pins under `root`, plants one mistake and runs
    the pins there; returns (returncode, stdout)."""
    for d in ("oracle", "tests", "zr_workloads"):
        shutil.copytree(os.path.join(ROOT, d), os.path.join(root, d),
                        ignore=shutil.ignore_patterns("*.so", "__pycache__"))
    target = os.path.join(root, path)
    with open(target) as f:
        text = f.read()
    if text.count(old) < 1:
        return None, f"mutation anchor not found: {old!r}"
    with open(target, "w") as f:
        f.write(text.replace(old, new))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", *PIN_TESTS],
                       cwd=root, capture_output=True, text=True, timeout=600)
    return r.returncode, r.stdout


_futures = {}


def _result(tmp_path_factory, what):
    """Outside pytest-xdist the first test starts every mutation at once on a
    few host cores; each test then waits for its own."""
    if os.environ.get("PYTEST_XDIST_WORKER"):
        m = next(x for x in MUTATIONS if x[0] == what)
        return _plant_and_run(str(tmp_path_factory.mktemp("mut")), *m)
    if not _futures:
        workers = max(2, len(os.sched_getaffinity(0)) // 2)
        pool = ThreadPoolExecutor(max_workers=workers)
        for m in MUTATIONS:
            _futures[m[0]] = pool.submit(_plant_and_run, str(tmp_path_factory.mktemp("mut")), *m)
        pool.shutdown(wait=False)
    return _futures[what].result()


@pytest.mark.parametrize("what", [m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(tmp_path_factory, what):
    code, out = _result(tmp_path_factory, what)
    assert code is not None, out
    assert code != 0, f"planted mistake '{what}' passed every pin:\n{out[-2000:]}"
    assert "failed" in out
