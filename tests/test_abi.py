"""CPU tests of the C ABI: every symbol zr.h declares is exported, the layout
queries equal the oracle bit for bit, and every validation path returns its
documented code without launching anything (no GPU is touched here)."""
import ctypes
import os
import random
import re

import pytest
import torch

import oracle
import zero_sharded_optimizer_zr_amd as zr
from zr_workloads import ALL, GPT_7P5B, LLAMA_7B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "zr.h")


def declared_functions():
    text = open(HEADER).read()
    return re.findall(r"^ZR_API\s+[\w\s\*]+?\b(zr_\w+)\s*\(", text, flags=re.M)


def test_every_declared_symbol_is_exported_and_bound():
    names = declared_functions()
    assert len(names) == 34
    lib = ctypes.CDLL(zr.LIBRARY)
    for name in names:
        assert hasattr(lib, name), name
        assert callable(getattr(zr, name)), name
        assert name in zr.__all__, name
    assert all(hasattr(zr, name) for name in zr.__all__)
    assert set(names) == set(zr.SYMBOLS)
    assert zr.zr_abi_version() == 1


def _compare_layout(numels, n_d, thr):
    ref = oracle.Layout(numels, n_d, thr)
    lay = zr.zr_layout_create(numels, n_d, thr)
    info = zr.zr_layout_query(lay)
    assert (info["psi"], info["psi_part"], info["psi_persist"], info["psi_pad"], info["shard"]) == \
        (ref.psi, ref.psi_part, ref.psi_persist, ref.psi_pad, ref.shard)
    assert (info["n_d"], info["n_tensors"], info["threshold"]) == (n_d, len(numels), thr)
    assert (info["n_partitioned"], info["n_persistent"]) == (ref.n_partitioned, ref.n_persistent)
    for t in range(len(numels)):
        assert zr.zr_layout_tensor(lay, t) == (ref.persistent[t], ref.offset[t])
    for r in range(n_d):
        assert zr.zr_layout_rank_range(lay, r) == ref.rank_range(r)
    for stage in range(4):
        assert zr.zr_layout_ledger_bytes(lay, stage) == ref.ledger_bytes(stage)
    return lay, ref


@pytest.mark.parametrize("seed", range(60))
def test_layout_matches_oracle_random(seed):
    rng = random.Random(seed)
    numels = [rng.choice([0, 1, 3, 7, 8, 9, 16, 100, rng.randrange(0, 5000)]) for _ in range(rng.randrange(0, 12))]
    n_d = rng.randrange(1, 70)
    thr = rng.choice([0, 1, 8, 100, 10**6])
    lay, ref = _compare_layout(numels, n_d, thr)
    ranges = [(0, ref.psi_pad)] + [ref.rank_range(r) for r in range(n_d)]
    for _ in range(20):
        b = rng.randrange(0, ref.psi_pad + 1)
        ranges.append((b, rng.randrange(b, ref.psi_pad + 1)))
    for b, e in ranges:
        assert zr.zr_layout_fragments(lay, b, e) == ref.fragments(b, e)


@pytest.mark.parametrize("w", ALL, ids=[w.name for w in ALL])
def test_layout_matches_oracle_on_workloads(w):
    lay, ref = _compare_layout(w.numels, w.n_d, w.threshold)
    b, e = ref.rank_range(w.rank)
    assert zr.zr_layout_fragments(lay, b, e) == ref.fragments(b, e)
    if len(w.numels) > 1:
        assert zr.zr_layout_fragments(lay, 0, ref.psi_pad) == ref.fragments(0, ref.psi_pad)


def test_workload_shapes():
    llama = oracle.Layout(LLAMA_7B.numels, 64)
    assert llama.psi == 6_738_415_616 and llama.shard == 105_283_584
    assert len(llama.fragments(*llama.rank_range(17))) == 4
    gpt = oracle.Layout(GPT_7P5B.numels, 64)
    assert gpt.psi == 7_455_727_616 and gpt.n_persistent == 290 and gpt.shard == 116_465_664


def test_fragment_capacity_two_call_idiom():
    lay = zr.zr_layout_create([5, 5, 5], 1, 0)
    n = ctypes.c_int32()
    st = zr._lib.zr_layout_fragments(lay.handle, 0, 15, None, 0, ctypes.byref(n))
    assert st == zr.ZR_ERANGE and n.value == 3
    buf = (zr._Fragment * 2)()
    st = zr._lib.zr_layout_fragments(lay.handle, 0, 15, buf, 2, ctypes.byref(n))
    assert st == zr.ZR_ERANGE and n.value == 3 and buf[1].tensor == 1


# ------------------------------------------------------------ validation ----

def _status(fn, *args):
    return fn(*args)


def test_layout_create_errors():
    L = zr._lib
    out = ctypes.c_void_p()
    arr = (ctypes.c_int64 * 2)(5, 6)
    assert L.zr_layout_create(arr, 2, 4, 0, None) == zr.ZR_EINVAL
    assert L.zr_layout_create(None, 2, 4, 0, ctypes.byref(out)) == zr.ZR_EINVAL
    assert L.zr_layout_create(arr, -1, 4, 0, ctypes.byref(out)) == zr.ZR_EINVAL
    assert L.zr_layout_create(arr, 2, 0, 0, ctypes.byref(out)) == zr.ZR_EINVAL
    assert "n_d" in zr.zr_last_error()
    assert L.zr_layout_create(arr, 2, 4, -1, ctypes.byref(out)) == zr.ZR_EINVAL
    neg = (ctypes.c_int64 * 2)(5, -6)
    assert L.zr_layout_create(neg, 2, 4, 0, ctypes.byref(out)) == zr.ZR_EINVAL
    huge = (ctypes.c_int64 * 2)(2**62, 2**62)
    assert L.zr_layout_create(huge, 2, 4, 0, ctypes.byref(out)) == zr.ZR_EINVAL
    assert "overflow" in zr.zr_last_error()
    # empty list and all-persistent list are valid: psi_pad = shard = 0
    lay = zr.zr_layout_create([], 4)
    assert zr.zr_layout_query(lay)["psi_pad"] == 0
    lay = zr.zr_layout_create([3, 4], 4, 100)
    assert zr.zr_layout_query(lay)["shard"] == 0 and zr.zr_layout_fragments(lay, 0, 0) == []
    L.zr_layout_destroy(None)


def test_layout_query_errors():
    lay = zr.zr_layout_create([10, 20], 4, 0)
    with pytest.raises(zr.ZRError) as e:
        zr.zr_layout_tensor(lay, 2)
    assert e.value.status == zr.ZR_ERANGE
    with pytest.raises(zr.ZRError) as e:
        zr.zr_layout_rank_range(lay, 4)
    assert e.value.status == zr.ZR_ERANGE
    with pytest.raises(zr.ZRError) as e:
        zr.zr_layout_rank_range(lay, -1)
    assert e.value.status == zr.ZR_ERANGE
    with pytest.raises(zr.ZRError) as e:
        zr.zr_layout_fragments(lay, 0, 33)
    assert e.value.status == zr.ZR_ERANGE
    with pytest.raises(zr.ZRError) as e:
        zr.zr_layout_fragments(lay, 5, 4)
    assert e.value.status == zr.ZR_ERANGE
    with pytest.raises(zr.ZRError) as e:
        zr.zr_layout_ledger_bytes(lay, 4)
    assert e.value.status == zr.ZR_ERANGE
    assert zr._lib.zr_layout_query(None, None) == zr.ZR_EINVAL


# fake, suitably aligned device addresses: validation must reject before any use
A = 0x7F0000000000


def _hp(**kw):
    base = dict(lr=5e-5, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, grad_scale=1.0, step=1)
    base.update(kw)
    return zr._HParams(**base)


@pytest.mark.parametrize("case,args,code", [
    ("null hp", (A, A + 2**20, A + 2**21, A + 2**22, A + 2**23, 16, None), zr.ZR_EINVAL),
    ("negative numel", (A, A + 2**20, A + 2**21, A + 2**22, A + 2**23, -1, "hp"), zr.ZR_EINVAL),
    ("null master", (A, None, A + 2**21, A + 2**22, A + 2**23, 16, "hp"), zr.ZR_EINVAL),
    ("step 0", (A, A + 2**20, A + 2**21, A + 2**22, A + 2**23, 16, _hp(step=0)), zr.ZR_EINVAL),
    ("beta1 = 1", (A, A + 2**20, A + 2**21, A + 2**22, A + 2**23, 16, _hp(beta1=1.0)), zr.ZR_EINVAL),
    ("beta2 < 0", (A, A + 2**20, A + 2**21, A + 2**22, A + 2**23, 16, _hp(beta2=-0.1)), zr.ZR_EINVAL),
    ("eps = 0", (A, A + 2**20, A + 2**21, A + 2**22, A + 2**23, 16, _hp(eps=0.0)), zr.ZR_EINVAL),
    ("lr nan", (A, A + 2**20, A + 2**21, A + 2**22, A + 2**23, 16, _hp(lr=float("nan"))), zr.ZR_EINVAL),
    ("wd < 0", (A, A + 2**20, A + 2**21, A + 2**22, A + 2**23, 16, _hp(weight_decay=-1.0)), zr.ZR_EINVAL),
    ("scale inf", (A, A + 2**20, A + 2**21, A + 2**22, A + 2**23, 16, _hp(grad_scale=float("inf"))), zr.ZR_EINVAL),
    ("odd grad", (A + 1, A + 2**20, A + 2**21, A + 2**22, A + 2**23, 16, "hp"), zr.ZR_EALIGN),
    ("master 2-aligned", (A, A + 2**20 + 2, A + 2**21, A + 2**22, A + 2**23, 16, "hp"), zr.ZR_EALIGN),
    ("m overlaps v", (A, A + 2**20, A + 2**21, A + 2**21 + 32, A + 2**23, 16, "hp"), zr.ZR_EINVAL),
    ("param overlaps grad", (A, A + 2**20, A + 2**21, A + 2**22, A + 16, 16, "hp"), zr.ZR_EINVAL),
])
def test_adamw_validation(case, args, code):
    *ptrs, numel, hp = args
    hp = _hp() if hp == "hp" else hp
    st = zr._lib.zr_adamw_step(*ptrs, numel, None if hp is None else ctypes.byref(hp), None)
    assert st == code, (case, zr.zr_last_error())
    assert zr.zr_last_error()


def test_adamw_empty_is_a_no_op():
    hp = _hp()
    assert zr._lib.zr_adamw_step(None, None, None, None, None, 0, ctypes.byref(hp), None) == zr.ZR_OK


def _table(*ptrs):
    return (ctypes.c_void_p * len(ptrs))(*ptrs)


@pytest.mark.parametrize("case,table,n,numel,out,code", [
    ("null table", None, 2, 16, A, zr.ZR_EINVAL),
    ("n = 0", "t2", 0, 16, A, zr.ZR_EINVAL),
    ("n = 257", "t2", 257, 16, A, zr.ZR_EINVAL),
    ("negative numel", "t2", 2, -5, A, zr.ZR_EINVAL),
    ("null out", "t2", 2, 16, None, zr.ZR_EINVAL),
    ("odd out", "t2", 2, 16, A + 1, zr.ZR_EALIGN),
    ("null contribution", "tnull", 2, 16, A, zr.ZR_EINVAL),
    ("odd contribution", "todd", 2, 16, A, zr.ZR_EALIGN),
    ("out overlaps contribs[1]", "t2", 2, 16, A + 2**20 + 4, zr.ZR_EINVAL),
    ("out inside contribs[0]", "t2", 2, 16, A + 2**21 + 2, zr.ZR_EINVAL),
])
def test_reduce_validation(case, table, n, numel, out, code):
    tables = {"t2": _table(A + 2**21, A + 2**20), "tnull": _table(A + 2**21, None),
              "todd": _table(A + 2**21, A + 2**20 + 1)}
    t = tables.get(table)
    # "n = 257" reads only the count, never the table entries
    st = zr._lib.zr_reduce_slice(t, n, numel, out, None)
    assert st == code, (case, zr.zr_last_error())


def test_reduce_empty_is_a_no_op():
    assert zr._lib.zr_reduce_slice(_table(A, A + 64), 2, 0, A + 128, None) == zr.ZR_OK


def _views(*entries):
    arr = (zr._View * len(entries))()
    for i, (p, first, count) in enumerate(entries):
        arr[i].ptr, arr[i].first, arr[i].count = p, first, count
    return arr


def test_pack_unpack_validation():
    lay = zr.zr_layout_create([10, 6, 3], 4, 4)  # tensor 2 (3 elements) persistent; psi_pad 16
    L = zr._lib
    good = _views((A, 0, 10), (A + 4096, 0, 6), (None, 0, 0))
    flat = A + 2**20
    for fn in ("pack", "unpack"):
        def call(layout, views, n_views, fl, b, e):
            if fn == "pack":
                return L.zr_pack(layout, views, n_views, fl, b, e, None)
            return L.zr_unpack(layout, fl, b, e, views, n_views, None)
        assert call(None, good, 3, flat, 0, 16) == zr.ZR_EINVAL
        assert call(lay.handle, good, 2, flat, 0, 16) == zr.ZR_EINVAL       # n_views != n_tensors
        assert call(lay.handle, None, 3, flat, 0, 16) == zr.ZR_EINVAL
        assert call(lay.handle, good, 3, flat, 0, 17) == zr.ZR_ERANGE       # beyond psi_pad
        assert call(lay.handle, good, 3, flat, 8, 4) == zr.ZR_ERANGE        # begin > end
        assert call(lay.handle, good, 3, flat, -1, 4) == zr.ZR_ERANGE
        assert call(lay.handle, good, 3, None, 0, 16) == zr.ZR_EINVAL
        assert call(lay.handle, good, 3, flat + 1, 0, 16) == zr.ZR_EALIGN
        assert call(lay.handle, good, 3, flat, 5, 5) == zr.ZR_OK            # empty range
        short = _views((A, 0, 9), (A + 4096, 0, 6), (None, 0, 0))
        assert call(lay.handle, short, 3, flat, 0, 16) == zr.ZR_ERANGE      # view misses element 9
        assert "tensor 0" in zr.zr_last_error()
        window = _views((A, 4, 6), (A + 4096, 0, 6), (None, 0, 0))
        assert call(lay.handle, window, 3, flat, 0, 16) == zr.ZR_ERANGE     # window starts too late
        missing = _views((A, 0, 10), (None, 0, 0), (None, 0, 0))
        assert call(lay.handle, missing, 3, flat, 0, 16) == zr.ZR_EINVAL
        odd = _views((A + 1, 0, 10), (A + 4096, 0, 6), (None, 0, 0))
        assert call(lay.handle, odd, 3, flat, 0, 16) == zr.ZR_EALIGN
        clash = _views((flat + 8, 0, 10), (A + 4096, 0, 6), (None, 0, 0))
        assert call(lay.handle, clash, 3, flat, 0, 16) == zr.ZR_EINVAL      # view overlaps flat


def test_binding_rejects_bad_tensors():
    lay = zr.zr_layout_create([10], 1, 0)
    with pytest.raises(TypeError):
        zr.zr_pack(lay, [torch.zeros(10, dtype=torch.float32)], torch.zeros(10, dtype=torch.int16), 0, 10, stream=0)
    with pytest.raises(ValueError):
        zr.zr_unpack(lay, torch.zeros(20, dtype=torch.int16)[::2], 0, 10, [torch.zeros(10, dtype=torch.int16)],
                     stream=0)


def test_binding_rejects_host_tensors_for_kernels():
    """Every wrapper of a GPU kernel refuses host (CPU) tensors of the right
    size and dtype with ValueError before the library is called, so a host
    address never reaches a kernel; the host AdamW refuses GPU-side roles the
    same way (no GPU is touched: every case fails in the binding)."""
    i16 = lambda n: torch.zeros(n, dtype=torch.int16)
    f32 = lambda n: torch.zeros(n, dtype=torch.float32)
    ls = torch.zeros(4, dtype=torch.int32)
    hp = dict(lr=5e-5, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, step=1)
    lay = zr.zr_layout_create([300_000, 200_000], 4)
    views = [i16(300_000), i16(200_000)]
    cases = {
        "pack": lambda: zr.zr_pack(lay, views, i16(100), 0, 100),
        "unpack": lambda: zr.zr_unpack(lay, i16(100), 0, 100, views),
        "reduce": lambda: zr.zr_reduce_slice([i16(100), i16(100)], i16(100)),
        "adamw": lambda: zr.zr_adamw_step(i16(100), f32(100), f32(100), f32(100), i16(100), **hp),
        "adamw no copy": lambda: zr.zr_adamw_step(i16(100), f32(100), f32(100), f32(100), None, **hp),
        "fused": lambda: zr.zr_reduce_adamw_step([i16(100)], f32(100), f32(100), f32(100), None, i16(100), **hp),
        "ls init": lambda: zr.zr_loss_scale_init(ls),
        "reduce f16": lambda: zr.zr_reduce_slice_f16([i16(100)], i16(100), ls),
        "check f16": lambda: zr.zr_check_finite_f16(i16(100), ls),
        "adamw f16": lambda: zr.zr_adamw_step_f16(i16(100), f32(100), f32(100), f32(100), None, ls, **hp),
        "ls update": lambda: zr.zr_loss_scale_update(ls),
        "quantize int8": lambda: zr.zr_quantize_int8(i16(100), torch.zeros(100, dtype=torch.int8), f32(1),
                                                     block=256),
        "dequantize int8": lambda: zr.zr_dequantize_int8(torch.zeros(100, dtype=torch.int8), f32(1), i16(100),
                                                         block=256),
        "unpack int8": lambda: zr.zr_unpack_int8(lay, torch.zeros(1000, dtype=torch.int8), f32(4), 0, 1000, views,
                                                 block=256),
        "quantize int4": lambda: zr.zr_quantize_int4(i16(100), torch.zeros(50, dtype=torch.uint8), f32(1),
                                                     block=256),
        "dequantize int4": lambda: zr.zr_dequantize_int4(torch.zeros(50, dtype=torch.uint8), f32(1), i16(100),
                                                         block=256),
        "unpack int4": lambda: zr.zr_unpack_int4(lay, torch.zeros(500, dtype=torch.uint8), f32(4), 0, 1000, views,
                                                 block=256),
    }
    for name, call in cases.items():
        with pytest.raises(ValueError, match="must be a cuda tensor"):
            call()
    # the offload step's gradient and parameters are device buffers
    staging = torch.zeros(1 << 16, dtype=torch.uint8)
    with pytest.raises(ValueError):
        zr.zr_offload_adamw_step(i16(100), f32(100), f32(100), f32(100), i16(100), staging, **hp)


@pytest.mark.parametrize("case,table,n,outs,numel,hp,code", [
    ("null hp", "t2", 2, (A, A + 2**24, A + 2**25, A + 2**26, None), 16, None, zr.ZR_EINVAL),
    ("null table", None, 2, (A, A + 2**24, A + 2**25, A + 2**26, None), 16, "hp", zr.ZR_EINVAL),
    ("n = 0", "t2", 0, (A, A + 2**24, A + 2**25, A + 2**26, None), 16, "hp", zr.ZR_EINVAL),
    ("n = 257", "t2", 257, (A, A + 2**24, A + 2**25, A + 2**26, None), 16, "hp", zr.ZR_EINVAL),
    ("negative numel", "t2", 2, (A, A + 2**24, A + 2**25, A + 2**26, None), -1, "hp", zr.ZR_EINVAL),
    ("null master", "t2", 2, (None, A + 2**24, A + 2**25, A + 2**26, None), 16, "hp", zr.ZR_EINVAL),
    ("step 0", "t2", 2, (A, A + 2**24, A + 2**25, A + 2**26, None), 16, _hp(step=0), zr.ZR_EINVAL),
    ("odd param", "t2", 2, (A, A + 2**24, A + 2**25, A + 2**26 + 1, None), 16, "hp", zr.ZR_EALIGN),
    ("m overlaps master", "t2", 2, (A, A + 32, A + 2**25, A + 2**26, None), 16, "hp", zr.ZR_EINVAL),
    ("grad_out overlaps v", "t2", 2, (A, A + 2**24, A + 2**25, A + 2**26, A + 2**25 + 8), 16, "hp", zr.ZR_EINVAL),
    ("contribution overlaps master", "tclash", 2, (A, A + 2**24, A + 2**25, A + 2**26, None), 16, "hp",
     zr.ZR_EINVAL),
    ("grad_out inside contribs[1]", "t2", 2, (A, A + 2**24, A + 2**25, A + 2**26, A + 2**28 + 4), 16, "hp",
     zr.ZR_EINVAL),
    ("odd contribution", "todd", 2, (A, A + 2**24, A + 2**25, A + 2**26, None), 16, "hp", zr.ZR_EALIGN),
])
def test_fused_validation(case, table, n, outs, numel, hp, code):
    tables = {"t2": _table(A + 2**27, A + 2**28), "tclash": _table(A + 2**27, A + 8),
              "todd": _table(A + 2**27, A + 2**28 + 1)}
    hp = _hp() if hp == "hp" else hp
    st = zr._lib.zr_reduce_adamw_step(tables.get(table), n, *outs[:4], outs[4], numel,
                                      None if hp is None else ctypes.byref(hp), None)
    assert st == code, (case, zr.zr_last_error())


def test_fused_empty_is_a_no_op():
    hp = _hp()
    assert zr._lib.zr_reduce_adamw_step(_table(A, A + 64), 2, None, None, None, None, None, 0,
                                        ctypes.byref(hp), None) == zr.ZR_OK


def test_fp16_validation():
    L = zr._lib
    hp = _hp()
    ls = A + 2**30
    # loss-scale record
    assert L.zr_loss_scale_init(None, 65536.0, None) == zr.ZR_EINVAL
    assert L.zr_loss_scale_init(ls + 2, 65536.0, None) == zr.ZR_EALIGN
    assert L.zr_loss_scale_init(ls, 0.0, None) == zr.ZR_EINVAL
    assert L.zr_loss_scale_init(ls, float("inf"), None) == zr.ZR_EINVAL
    assert L.zr_loss_scale_update(ls, 0, 2.0, 1.0, None) == zr.ZR_EINVAL
    assert L.zr_loss_scale_update(ls, 1000, 1.0, 1.0, None) == zr.ZR_EINVAL
    assert L.zr_loss_scale_update(ls, 1000, 2.0, 0.0, None) == zr.ZR_EINVAL
    assert L.zr_loss_scale_update(None, 1000, 2.0, 1.0, None) == zr.ZR_EINVAL
    # finite check
    assert L.zr_check_finite_f16(A, 16, None, None) == zr.ZR_EINVAL
    assert L.zr_check_finite_f16(A + 1, 16, ls, None) == zr.ZR_EALIGN
    assert L.zr_check_finite_f16(ls - 8, 16, ls, None) == zr.ZR_EINVAL     # record inside grad
    assert L.zr_check_finite_f16(A, -1, ls, None) == zr.ZR_EINVAL
    assert L.zr_check_finite_f16(None, 0, ls, None) == zr.ZR_OK
    # fp16 mean
    t = _table(A + 2**21, A + 2**20)
    assert L.zr_reduce_slice_f16(t, 0, 16, A, None, None) == zr.ZR_EINVAL
    assert L.zr_reduce_slice_f16(t, 2, 16, A + 1, None, None) == zr.ZR_EALIGN
    assert L.zr_reduce_slice_f16(t, 2, 16, A, ls + 1, None) == zr.ZR_EALIGN
    assert L.zr_reduce_slice_f16(t, 2, 16, A + 2**20 + 4, None, None) == zr.ZR_EINVAL
    assert L.zr_reduce_slice_f16(t, 2, 16, A, A + 2**21 + 8, None) == zr.ZR_EINVAL   # record inside a contribution
    assert L.zr_reduce_slice_f16(t, 2, 0, A, None, None) == zr.ZR_OK
    # loss-scaled AdamW
    args = (A, A + 2**22, A + 2**23, A + 2**24, A + 2**25)
    assert L.zr_adamw_step_f16(*args, 16, ctypes.byref(hp), None, None) == zr.ZR_EINVAL
    assert L.zr_adamw_step_f16(*args, 16, None, ls, None) == zr.ZR_EINVAL
    assert L.zr_adamw_step_f16(*args, 16, ctypes.byref(_hp(step=0)), ls, None) == zr.ZR_EINVAL
    assert L.zr_adamw_step_f16(A, A + 2**22 + 2, *args[2:], 16, ctypes.byref(hp), ls, None) == zr.ZR_EALIGN
    assert L.zr_adamw_step_f16(*args, 16, ctypes.byref(hp), A + 2**23 + 16, None) == zr.ZR_EINVAL  # record in m
    assert L.zr_adamw_step_f16(*args, 0, ctypes.byref(hp), ls, None) == zr.ZR_OK


def test_int8_validation():
    L = zr._lib
    src, q, sc, dst = A, A + 2**22, A + 2**23, A + 2**24
    for block in (0, 1, 128, 300, 4096, -256):
        assert L.zr_quantize_int8(src, 1000, block, q, sc, None) == zr.ZR_EINVAL
        assert L.zr_dequantize_int8(q, sc, 1000, block, dst, None) == zr.ZR_EINVAL
    assert L.zr_quantize_int8(src, -1, 256, q, sc, None) == zr.ZR_EINVAL
    assert L.zr_quantize_int8(None, 16, 256, q, sc, None) == zr.ZR_EINVAL
    assert L.zr_quantize_int8(src, 16, 256, None, sc, None) == zr.ZR_EINVAL
    assert L.zr_quantize_int8(src, 16, 256, q, None, None) == zr.ZR_EINVAL
    assert L.zr_quantize_int8(src + 1, 16, 256, q, sc, None) == zr.ZR_EALIGN
    assert L.zr_quantize_int8(src, 16, 256, q, sc + 2, None) == zr.ZR_EALIGN
    assert L.zr_quantize_int8(src, 1000, 256, src + 1000, sc, None) == zr.ZR_EINVAL     # codes inside src
    assert L.zr_quantize_int8(src, 1000, 256, q, q + 996, None) == zr.ZR_EINVAL         # scales over the codes' tail
    assert L.zr_quantize_int8(src, 0, 256, q, sc, None) == zr.ZR_OK
    assert L.zr_quantize_int8(None, 0, 256, None, None, None) == zr.ZR_OK
    assert L.zr_dequantize_int8(q, sc, -1, 256, dst, None) == zr.ZR_EINVAL
    assert L.zr_dequantize_int8(q, sc, 16, 256, None, None) == zr.ZR_EINVAL
    assert L.zr_dequantize_int8(None, sc, 16, 256, dst, None) == zr.ZR_EINVAL
    assert L.zr_dequantize_int8(q, sc, 16, 256, dst + 1, None) == zr.ZR_EALIGN
    assert L.zr_dequantize_int8(q, sc + 1, 16, 256, dst, None) == zr.ZR_EALIGN
    assert L.zr_dequantize_int8(q, sc, 1000, 256, q - 1000, None) == zr.ZR_EINVAL       # dst over the codes' head
    assert L.zr_dequantize_int8(q, sc, 0, 256, dst, None) == zr.ZR_OK



def test_int4_validation():
    L = zr._lib
    src, q, sc, dst = A, A + 2**22, A + 2**23, A + 2**24
    for block in (0, 1, 128, 300, 4096, -256):
        assert L.zr_quantize_int4(src, 1000, block, q, sc, None) == zr.ZR_EINVAL
        assert L.zr_dequantize_int4(q, sc, 1000, block, dst, None) == zr.ZR_EINVAL
    assert L.zr_quantize_int4(src, -1, 256, q, sc, None) == zr.ZR_EINVAL
    assert L.zr_quantize_int4(None, 16, 256, q, sc, None) == zr.ZR_EINVAL
    assert L.zr_quantize_int4(src, 16, 256, None, sc, None) == zr.ZR_EINVAL
    assert L.zr_quantize_int4(src, 16, 256, q, None, None) == zr.ZR_EINVAL
    assert L.zr_quantize_int4(src + 1, 16, 256, q, sc, None) == zr.ZR_EALIGN
    assert L.zr_quantize_int4(src, 16, 256, q, sc + 2, None) == zr.ZR_EALIGN
    assert L.zr_quantize_int4(src, 1000, 256, src + 1000, sc, None) == zr.ZR_EINVAL     # codes inside src
    assert L.zr_quantize_int4(src, 1000, 256, q, q + 496, None) == zr.ZR_EINVAL         # scales over the codes' tail
    assert L.zr_quantize_int4(src, 0, 256, q, sc, None) == zr.ZR_OK
    assert L.zr_quantize_int4(None, 0, 256, None, None, None) == zr.ZR_OK
    assert L.zr_dequantize_int4(q, sc, -1, 256, dst, None) == zr.ZR_EINVAL
    assert L.zr_dequantize_int4(q, sc, 16, 256, None, None) == zr.ZR_EINVAL
    assert L.zr_dequantize_int4(None, sc, 16, 256, dst, None) == zr.ZR_EINVAL
    assert L.zr_dequantize_int4(q, sc, 16, 256, dst + 1, None) == zr.ZR_EALIGN
    assert L.zr_dequantize_int4(q, sc + 1, 16, 256, dst, None) == zr.ZR_EALIGN
    assert L.zr_dequantize_int4(q, sc, 1000, 256, q - 1000, None) == zr.ZR_EINVAL       # dst over the codes' head
    assert L.zr_dequantize_int4(q, sc, 0, 256, dst, None) == zr.ZR_OK


def test_int4_binding_checks_buffer_sizes():
    src = torch.zeros(1001, dtype=torch.int16)
    with pytest.raises(ValueError):   # 1001 codes need 501 bytes
        zr.zr_quantize_int4(src, torch.zeros(500, dtype=torch.uint8), torch.zeros(4, dtype=torch.float32), block=256)
    with pytest.raises(ValueError):
        zr.zr_quantize_int4(src, torch.zeros(501, dtype=torch.uint8), torch.zeros(3, dtype=torch.float32), block=256)
    with pytest.raises(ValueError):
        zr.zr_dequantize_int4(torch.zeros(501, dtype=torch.uint8), torch.zeros(1, dtype=torch.float32), src, block=512)


def test_int8_binding_checks_buffer_sizes():
    src = torch.zeros(1000, dtype=torch.int16)
    with pytest.raises(ValueError):
        zr.zr_quantize_int8(src, torch.zeros(999, dtype=torch.int8), torch.zeros(4, dtype=torch.float32), block=256)
    with pytest.raises(ValueError):
        zr.zr_quantize_int8(src, torch.zeros(1000, dtype=torch.int8), torch.zeros(3, dtype=torch.float32), block=256)
    with pytest.raises(TypeError):
        zr.zr_quantize_int8(src, torch.zeros(1000, dtype=torch.int16), torch.zeros(4, dtype=torch.float32), block=256)
    with pytest.raises(ValueError):
        zr.zr_dequantize_int8(torch.zeros(1000, dtype=torch.int8), torch.zeros(1, dtype=torch.float32), src, block=512)


@pytest.mark.parametrize("fn", ["zr_unpack_int8", "zr_unpack_int4"])
def test_unpack_quantized_validation(fn):
    lay = zr.zr_layout_create([10, 6, 3], 4, 4)  # tensor 2 persistent; psi_pad 16, shard 4
    L = zr._lib
    good = _views((A, 0, 10), (A + 4096, 0, 6), (None, 0, 0))
    q, sc = A + 2**20, A + 2**21
    code_bytes = 16 if fn == "zr_unpack_int8" else 8   # int4: 2 bytes per shard of 4

    def call(layout, qq, ss, block, b, e, views=good, n_views=3):
        return getattr(L, fn)(layout, qq, ss, block, b, e, views, n_views, None)

    assert call(None, q, sc, 256, 0, 16) == zr.ZR_EINVAL
    for block in (0, 128, 300, 4096):
        assert call(lay.handle, q, sc, block, 0, 16) == zr.ZR_EINVAL
    assert call(lay.handle, q, sc, 256, 0, 17) == zr.ZR_ERANGE
    assert call(lay.handle, q, sc, 256, 9, 4) == zr.ZR_ERANGE
    assert call(lay.handle, q, sc, 256, 0, 16, n_views=2) == zr.ZR_EINVAL
    assert call(lay.handle, q, sc, 256, 0, 16, views=None) == zr.ZR_EINVAL
    assert call(lay.handle, None, sc, 256, 0, 16) == zr.ZR_EINVAL
    assert call(lay.handle, q, None, 256, 0, 16) == zr.ZR_EINVAL
    assert call(lay.handle, q, sc + 2, 256, 0, 16) == zr.ZR_EALIGN
    assert call(lay.handle, q, q + code_bytes - 4, 256, 0, 16) == zr.ZR_EINVAL   # scales over the codes' tail
    assert call(lay.handle, q, sc, 256, 3, 3) == zr.ZR_OK                   # empty range
    assert call(lay.handle, None, None, 256, 3, 3) == zr.ZR_OK
    short = _views((A, 0, 9), (A + 4096, 0, 6), (None, 0, 0))
    assert call(lay.handle, q, sc, 256, 0, 16, views=short) == zr.ZR_ERANGE
    missing = _views((A, 0, 10), (None, 0, 0), (None, 0, 0))
    assert call(lay.handle, q, sc, 256, 0, 16, views=missing) == zr.ZR_EINVAL
    odd = _views((A + 1, 0, 10), (A + 4096, 0, 6), (None, 0, 0))
    assert call(lay.handle, q, sc, 256, 0, 16, views=odd) == zr.ZR_EALIGN
    over_q = _views((q + 4, 0, 10), (A + 4096, 0, 6), (None, 0, 0))
    assert call(lay.handle, q, sc, 256, 0, 16, views=over_q) == zr.ZR_EINVAL
    over_s = _views((A, 0, 10), (sc - 4, 0, 6), (None, 0, 0))
    assert call(lay.handle, q, sc, 256, 0, 16, views=over_s) == zr.ZR_EINVAL


def test_binding_rejects_short_tensors():
    """Every wrapper checks that each tensor holds the count it is asked to
    process before anything reaches the library (no GPU is touched)."""
    i16 = lambda n: torch.zeros(n, dtype=torch.int16)
    f32 = lambda n: torch.zeros(n, dtype=torch.float32)
    hp = dict(lr=5e-5, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, step=1)
    lay = zr.zr_layout_create([300_000, 200_000], 4)
    cases = [
        lambda: zr.zr_pack(lay, [i16(300_000), i16(200_000)], i16(99), 0, 100),
        lambda: zr.zr_unpack(lay, i16(99), 0, 100, [i16(300_000), i16(200_000)]),
        lambda: zr.zr_reduce_slice([i16(100), i16(99)], i16(100)),
        lambda: zr.zr_adamw_step(i16(99), f32(100), f32(100), f32(100), i16(100), **hp),
        lambda: zr.zr_adamw_step(i16(100), f32(100), f32(99), f32(100), None, **hp),
        lambda: zr.zr_adamw_step(i16(100), f32(100), f32(100), f32(100), i16(99), **hp),
        lambda: zr.zr_reduce_adamw_step([i16(100), i16(99)], f32(100), f32(100), f32(100), None, **hp),
        lambda: zr.zr_reduce_adamw_step([i16(100)], f32(100), f32(100), f32(100), None, i16(99), **hp),
        lambda: zr.zr_reduce_slice_f16([i16(99)], i16(100)),
        lambda: zr.zr_check_finite_f16(i16(99), torch.zeros(4, dtype=torch.int32), numel=100),
        lambda: zr.zr_adamw_step_f16(i16(99), f32(100), f32(100), f32(100), None,
                                     torch.zeros(4, dtype=torch.int32), **hp),
        lambda: zr.zr_quantize_int8(i16(99), torch.zeros(100, dtype=torch.int8), f32(1), block=256, numel=100),
        lambda: zr.zr_dequantize_int8(torch.zeros(100, dtype=torch.int8), f32(1), i16(99), block=256, numel=100),
        lambda: zr.zr_unpack_int8(lay, torch.zeros(999, dtype=torch.int8), f32(100), 0, 1000,
                                  [i16(300_000), i16(200_000)], block=256),
        # [124_900, 125_100) crosses the first shard edge: 2 blocks of 256 on each side -> 3 scales
        lambda: zr.zr_unpack_int8(lay, torch.zeros(200, dtype=torch.int8), f32(2), 124_900, 125_100,
                                  [i16(300_000), i16(200_000)], block=256),
        lambda: zr.zr_host_adamw_step(i16(100), f32(100), f32(100), f32(99), None, **hp),
    ]
    for k, call in enumerate(cases):
        with pytest.raises(ValueError):
            call()


def test_graph_validation():
    L = zr._lib
    hp = _hp()
    assert L.zr_graph_capture_begin(None) == zr.ZR_EINVAL
    assert L.zr_graph_capture_end(None, None) == zr.ZR_EINVAL
    assert L.zr_graph_info(None, None, None) == zr.ZR_EINVAL
    assert L.zr_graph_set_adamw(None, ctypes.byref(hp)) == zr.ZR_EINVAL
    assert L.zr_graph_launch(None, None) == zr.ZR_EINVAL
    L.zr_graph_destroy(None)
