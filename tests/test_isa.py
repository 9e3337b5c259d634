"""The gfx950 code of the streaming kernels has the shape their design states
(CPU only: hipcc cross-compiles the device code to assembly here).

For each hot kernel: every HBM access is a global (not flat) non-temporal load
or store of the stated width, there is no LDS instruction (the residency caps
reserve LDS but never touch it) and no scratch memory, and the number of
vector memory instructions in the body is the one the data layout implies."""
import os
import re
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.join(ROOT, "zero_sharded_optimizer_zr_amd"))
import build as zr_build  # noqa: E402

CSRC = os.path.join(ROOT, "zero_sharded_optimizer_zr_amd", "csrc")

# (source, mangled-name fragment, {instruction: count in the body}).  The
# counts are static instructions of the kernel body; the head/tail element
# paths use narrow accesses, which are not pinned.
#   AdamW: dwordx4 in/out of master, m, v; dwordx2 of gradient in, copy out.
#   reduce (8-pointer table): two batches of 4 contribution loads;
#   for 7-8 contributions: 8 eight-byte loads at once, one eight-byte store.
#   fused: master/m/v as AdamW, dwordx2 contribution loads (one batch of up to
#   8 in flight; its 8 guarded loads appear twice in the compiled body), dwordx2
#   copy.
#   copy: aligned or funnel-shifted (two) loads, one store per lane.
#   int8 quantizer: 4 chunks of 16-byte loads per tile, 8-byte code stores
#   (int4: 4-byte code stores, beside the scale stores of the same width).
#   int8 / int4 unpack: the 16-byte stores of the rebuilt chunks (two per lane;
#   int4 two or four) over the instantiations (code phase, whole tile, one scale
#   per chunk), as compiled; a change of the count is a change of the kernel's
#   shape.
KERNELS = [
    ("adamw.hip", "adamw_vec_kernelILb1E", {"global_load_dwordx4": 3, "global_store_dwordx4": 3,
                                            "global_load_dwordx2": 1, "global_store_dwordx2": 1}),
    ("reduce.hip", "reduce_vec_kernelILi8EE", {"global_load_dwordx4": 8, "global_store_dwordx4": 1}),
    ("reduce.hip", "reduce4_vec_kernel", {"global_load_dwordx2": 8, "global_store_dwordx2": 1}),
    ("fused.hip", "fused_vec_kernelILi8ELb1ELb0E", {"global_load_dwordx4": 3, "global_store_dwordx4": 3,
                                                    "global_load_dwordx2": 16, "global_store_dwordx2": 1}),
    ("fp16.hip", "adamw_f16_vec_kernelILb1E", {"global_load_dwordx4": 3, "global_store_dwordx4": 3,
                                               "global_load_dwordx2": 1, "global_store_dwordx2": 1}),
    ("fp16.hip", "reduce4_f16_vec_kernel", {"global_load_dwordx2": 8, "global_store_dwordx2": 1}),
    ("copy.hip", "copy_kernel", {"global_load_dwordx4": 2, "global_store_dwordx4": 1}),
    ("unpack_quant.hip", "unpack_int8_kernel", {"global_store_dwordx4": 9}),
    ("quant.hip", "quantize_vec_kernelILi2048ELi127E", {"global_load_dwordx4": 4, "global_store_dwordx2": 4}),
    ("quant.hip", "quantize_vec_kernelILi2048ELi7E", {"global_load_dwordx4": 4}),
    ("quant.hip", "dequantize_vec_kernelILi2048ELi7E", {"global_store_dwordx4": 4}),
    ("unpack_quant.hip", "unpack_int4_kernelILi2ELi0E", {"global_store_dwordx4": 9}),
    ("unpack_quant.hip", "unpack_int4_kernelILi4ELi1E", {"global_store_dwordx4": 25}),
]


@pytest.fixture(scope="module")
def asm():
    """Device assembly of each source, compiled with the library's flags."""
    tmp = tempfile.mkdtemp(prefix="zr_isa_")
    files = sorted({k[0] for k in KERNELS})

    def compile_one(name):
        out = os.path.join(tmp, name + ".s")
        cmd = ["hipcc", *zr_build.FLAGS, f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
               "--offload-device-only", "-S", os.path.join(CSRC, name), "-o", out]
        r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
        assert r.returncode == 0, r.stderr[-2000:]
        with open(out) as f:
            return name, f.read()

    with ThreadPoolExecutor(len(files)) as pool:
        return dict(pool.map(compile_one, files))


def kernel_body(text, fragment):
    """Instructions between the kernel's entry label and the end of its
    function, and its metadata block."""
    m = re.search(r"^(_Z\S*" + re.escape(fragment) + r"\S*):", text, re.M)
    assert m, f"kernel {fragment} not found"
    name = m.group(1)
    start = m.end()
    end = text.index(".Lfunc_end", start)
    body = [ln.split(";")[0].strip() for ln in text[start:end].splitlines()]
    meta = text[text.index(f".name:           {name}"):]
    meta = meta[:meta.index("\n  - ") if "\n  - " in meta else len(meta)]
    return [ln for ln in body if ln and not ln.startswith(".")], meta


@pytest.mark.parametrize("src,frag,counts", KERNELS, ids=[k[1] for k in KERNELS])
def test_kernel_shape(asm, src, frag, counts):
    body, meta = kernel_body(asm[src], frag)
    ops = [ln.split()[0] for ln in body]
    assert not [o for o in ops if o.startswith("ds_")], "LDS instruction in a streaming kernel"
    assert not [o for o in ops if o.startswith(("scratch_", "buffer_"))], "scratch or buffer access"
    assert not [o for o in ops if o.startswith(("flat_load", "flat_store"))], "flat access (not global)"
    assert not [o for o in ops if o.startswith(("s_store", "s_buffer_store", "s_atomic", "s_buffer_atomic",
                                               "s_dcache_wb", "s_dcache_discard"))], "scalar-cache write"
    assert re.search(r"\.private_segment_fixed_size:\s+0\b", meta), "kernel uses scratch memory"
    for op, want in counts.items():
        lines = [ln for ln in body if ln.split()[0] == op]
        assert len(lines) == want, f"{op}: {len(lines)} in the body, expected {want}"
        assert all(ln.rstrip().endswith(" nt") for ln in lines), f"{op} without the non-temporal hint"
    wide = [ln for ln in body if ln.split()[0] in ("global_load_dwordx4", "global_store_dwordx4",
                                                   "global_load_dwordx2", "global_store_dwordx2")]
    assert wide, "no 8- or 16-byte global access"


def test_int4_dequantize_issues_its_loads_first(asm):
    """The int4 dequantizer's whole-tile path issues the code loads of all 4
    chunks of a lane before its first store (codes and output may alias for
    the compiler, so a load after a store would wait for it)."""
    body, _ = kernel_body(asm["quant.hip"], "dequantize_vec_kernelILi2048ELi7E")
    ops = [ln.split()[0] for ln in body]
    first_store = ops.index("global_store_dwordx4")
    assert ops[:first_store].count("global_load_dword") >= 4, ops[:first_store]
