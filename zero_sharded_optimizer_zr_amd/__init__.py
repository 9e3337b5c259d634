"""Python binding of libzr: one data-parallel rank's share of a ZeRO-3 step on
an AMD Instinct MI355X.

Argument marshalling only.  Every function has the name of the C entry point
it calls (declared in ``include/zr.h``); every step of the path runs in the
library's HIP kernels.  PyTorch provides device memory (``torch.Tensor``) and
streams.  Importing fails loudly if ``libzr.so`` has not been built.

bf16 buffers may be any 2-byte dtype (torch.bfloat16, torch.int16, ...); their
bits are passed through unchanged.  Every wrapper of a GPU kernel checks,
before the library is called, that its buffers are GPU tensors on the device
of the stream it enqueues on (ValueError otherwise).
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence, Tuple, Union

import torch  # loads the process's HIP runtime before libzr binds to it

__all__ = [
    "ZRError", "Layout", "Graph", "zr_layout_create", "zr_layout_destroy", "zr_layout_query", "zr_layout_tensor",
    "zr_layout_rank_range", "zr_layout_fragments", "zr_layout_ledger_bytes", "zr_pack", "zr_unpack",
    "zr_reduce_slice", "zr_adamw_step", "zr_reduce_adamw_step", "zr_loss_scale_init", "zr_reduce_slice_f16",
    "zr_check_finite_f16", "zr_adamw_step_f16", "zr_loss_scale_update", "loss_scale_record",
    "zr_quantize_int8", "zr_dequantize_int8", "zr_unpack_int8", "zr_quantize_int4", "zr_dequantize_int4",
    "zr_unpack_int4", "zr_host_simd", "zr_host_adamw_step", "offload_staging", "zr_offload_adamw_step",
    "zr_graph_capture_begin", "zr_graph_capture_end", "zr_graph_info", "zr_graph_set_adamw", "zr_graph_launch",
    "zr_graph_destroy", "zr_last_error", "zr_abi_version", "LIBRARY", "SYMBOLS",
]

LIBRARY = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libzr.so")

if not os.path.exists(LIBRARY):
    raise ImportError(f"{LIBRARY} is missing: build it first (python -c 'import __graft_entry__ as g; g.build()')")

_lib = ctypes.CDLL(LIBRARY)

ZR_OK, ZR_EINVAL, ZR_ERANGE, ZR_EALIGN, ZR_ENOMEM, ZR_EHIP = range(6)
_NAMES = {1: "ZR_EINVAL", 2: "ZR_ERANGE", 3: "ZR_EALIGN", 4: "ZR_ENOMEM", 5: "ZR_EHIP"}


class ZRError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_NAMES.get(status, status)}: {message}")
        self.status = status


class _Info(ctypes.Structure):
    _fields_ = [("psi", ctypes.c_int64), ("psi_part", ctypes.c_int64), ("psi_persist", ctypes.c_int64),
                ("psi_pad", ctypes.c_int64), ("shard", ctypes.c_int64), ("threshold", ctypes.c_int64),
                ("n_d", ctypes.c_int32), ("n_tensors", ctypes.c_int32), ("n_partitioned", ctypes.c_int32),
                ("n_persistent", ctypes.c_int32)]


class _Fragment(ctypes.Structure):
    _fields_ = [("tensor", ctypes.c_int32), ("reserved", ctypes.c_int32), ("tensor_offset", ctypes.c_int64),
                ("flat_offset", ctypes.c_int64), ("numel", ctypes.c_int64)]


class _View(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_void_p), ("first", ctypes.c_int64), ("count", ctypes.c_int64)]


class _HParams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_double), ("beta1", ctypes.c_double), ("beta2", ctypes.c_double),
                ("eps", ctypes.c_double), ("weight_decay", ctypes.c_double), ("grad_scale", ctypes.c_double),
                ("step", ctypes.c_int64)]


_P, _I32, _I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
_SIGS = {
    "zr_layout_create": ([_P, _I32, _I32, _I64, _P], _I32),
    "zr_layout_destroy": ([_P], None),
    "zr_layout_query": ([_P, _P], _I32),
    "zr_layout_tensor": ([_P, _I32, _P, _P], _I32),
    "zr_layout_rank_range": ([_P, _I32, _P, _P], _I32),
    "zr_layout_fragments": ([_P, _I64, _I64, _P, _I32, _P], _I32),
    "zr_layout_ledger_bytes": ([_P, _I32, _P], _I32),
    "zr_pack": ([_P, _P, _I32, _P, _I64, _I64, _P], _I32),
    "zr_unpack": ([_P, _P, _I64, _I64, _P, _I32, _P], _I32),
    "zr_reduce_slice": ([_P, _I32, _I64, _P, _P], _I32),
    "zr_adamw_step": ([_P, _P, _P, _P, _P, _I64, _P, _P], _I32),
    "zr_reduce_adamw_step": ([_P, _I32, _P, _P, _P, _P, _P, _I64, _P, _P], _I32),
    "zr_loss_scale_init": ([_P, ctypes.c_float, _P], _I32),
    "zr_reduce_slice_f16": ([_P, _I32, _I64, _P, _P, _P], _I32),
    "zr_check_finite_f16": ([_P, _I64, _P, _P], _I32),
    "zr_adamw_step_f16": ([_P, _P, _P, _P, _P, _I64, _P, _P, _P], _I32),
    "zr_loss_scale_update": ([_P, _I32, ctypes.c_float, ctypes.c_float, _P], _I32),
    "zr_quantize_int8": ([_P, _I64, _I32, _P, _P, _P], _I32),
    "zr_dequantize_int8": ([_P, _P, _I64, _I32, _P, _P], _I32),
    "zr_unpack_int8": ([_P, _P, _P, _I32, _I64, _I64, _P, _I32, _P], _I32),
    "zr_quantize_int4": ([_P, _I64, _I32, _P, _P, _P], _I32),
    "zr_dequantize_int4": ([_P, _P, _I64, _I32, _P, _P], _I32),
    "zr_unpack_int4": ([_P, _P, _P, _I32, _I64, _I64, _P, _I32, _P], _I32),
    "zr_host_adamw_step": ([_P, _P, _P, _P, _P, _I64, _P, _I32], _I32),
    "zr_host_simd": ([], ctypes.c_char_p),
    "zr_offload_adamw_step": ([_P, _P, _P, _P, _P, _I64, _P, _P, _I64, _I32, _P], _I32),
    "zr_graph_capture_begin": ([_P], _I32),
    "zr_graph_capture_end": ([_P, _P], _I32),
    "zr_graph_info": ([_P, _P, _P], _I32),
    "zr_graph_set_adamw": ([_P, _P], _I32),
    "zr_graph_launch": ([_P, _P], _I32),
    "zr_graph_destroy": ([_P], None),
    "zr_last_error": ([], ctypes.c_char_p),
    "zr_abi_version": ([], _I32),
}
for _name, (_args, _res) in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.argtypes = _args
    _f.restype = _res

SYMBOLS = tuple(_SIGS)


def zr_last_error() -> str:
    return _lib.zr_last_error().decode()


def zr_abi_version() -> int:
    return _lib.zr_abi_version()


def _check(status: int):
    if status != ZR_OK:
        raise ZRError(status, zr_last_error())


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _ptr(t: Optional[torch.Tensor], size: int, name: str, device: Optional[str] = None) -> Optional[int]:
    """Address of a contiguous tensor of `size`-byte elements; with `device`
    given, the tensor must also live there ("cpu" for the host AdamW's
    buffers).  The buffers of GPU kernels are checked by _gpu_call."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.element_size() != size:
        raise TypeError(f"{name} must have {size}-byte elements")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device.type != device:
        raise ValueError(f"{name} must be a {device} tensor, not one on {t.device}")
    return t.data_ptr() or None


def _one_gpu(stream, *tensors) -> None:
    """Every tensor among `tensors` (None skipped, lists of tensors or of
    (tensor, first) views flattened) must be a GPU tensor, and all of them on
    one device, the device of the stream the call is enqueued on (torch's
    current device when `stream` is None; a raw stream handle is taken to
    belong to that device).  A host address reaching a kernel would be a GPU
    memory fault, so it raises here, before the library is called."""
    flat = []
    for t in tensors:
        if isinstance(t, (list, tuple)):
            flat.extend(x[0] if isinstance(x, tuple) else x for x in t)
        else:
            flat.append(t)
    flat = [t for t in flat if isinstance(t, torch.Tensor)]
    for t in flat:
        if t.device.type != "cuda":
            raise ValueError(f"every buffer of a GPU kernel must be a cuda tensor, not one on {t.device}")
    devs = {t.device.index for t in flat}
    if len(devs) > 1:
        raise ValueError(f"tensors on several GPUs {sorted(devs)}: one call runs on one device")
    if not devs:
        return
    if isinstance(stream, torch.cuda.Stream):
        want = stream.device.index
    elif stream is None:
        want = torch.cuda.current_device()
    else:
        return
    if want not in devs:
        raise ValueError(f"tensors on cuda:{devs.pop()} but the stream is on cuda:{want}")


def _gpu_call(fn, stream, tensors, *args) -> None:
    """fn(*args, stream) after _one_gpu(stream, *tensors).  The caller has
    marshalled the arguments (checking sizes and dtypes) before the device
    check runs; the stream handle is resolved after it."""
    _one_gpu(stream, *tensors)
    _check(fn(*args, _stream(stream)))


def _need(n: int, **tensors):
    """Every given tensor (None skipped) must hold at least n elements: the
    library trusts the counts it is given, so a short tensor would mean an
    access past its end on the device."""
    for name, t in tensors.items():
        if t is not None and t.numel() < n:
            raise ValueError(f"{name} holds {t.numel()} elements, {n} needed")


# ---------------------------------------------------------------- layout ----

class Layout:
    """Owns a zr_layout handle (released on garbage collection)."""

    def __init__(self, handle: int, numels: Sequence[int]):
        self._h = ctypes.c_void_p(handle)
        self.numels = list(numels)

    @property
    def handle(self):
        return self._h

    def __del__(self):
        # at interpreter exit the module's globals may already be gone
        if getattr(self, "_h", None) and self._h.value and _lib is not None:
            _lib.zr_layout_destroy(self._h)
            self._h = ctypes.c_void_p(None)

    def info(self) -> dict:
        return zr_layout_query(self)


def zr_layout_create(numels: Sequence[int], n_d: int, persist_threshold: int = 100_000) -> Layout:
    arr = (ctypes.c_int64 * max(1, len(numels)))(*[int(x) for x in numels])
    out = ctypes.c_void_p()
    _check(_lib.zr_layout_create(arr, len(numels), int(n_d), int(persist_threshold), ctypes.byref(out)))
    return Layout(out.value, numels)


def zr_layout_destroy(layout: Layout) -> None:
    layout.__del__()


def zr_layout_query(layout: Layout) -> dict:
    info = _Info()
    _check(_lib.zr_layout_query(layout.handle, ctypes.byref(info)))
    return {name: getattr(info, name) for name, _ in _Info._fields_}


def zr_layout_tensor(layout: Layout, t: int) -> Tuple[bool, int]:
    p, off = ctypes.c_int32(), ctypes.c_int64()
    _check(_lib.zr_layout_tensor(layout.handle, int(t), ctypes.byref(p), ctypes.byref(off)))
    return bool(p.value), off.value


def zr_layout_rank_range(layout: Layout, rank: int) -> Tuple[int, int]:
    b, e = ctypes.c_int64(), ctypes.c_int64()
    _check(_lib.zr_layout_rank_range(layout.handle, int(rank), ctypes.byref(b), ctypes.byref(e)))
    return b.value, e.value


def zr_layout_fragments(layout: Layout, begin: int, end: int) -> List[Tuple[int, int, int, int]]:
    """(tensor, tensor_offset, flat_offset, numel) of every piece in [begin, end)."""
    n = ctypes.c_int32()
    status = _lib.zr_layout_fragments(layout.handle, int(begin), int(end), None, 0, ctypes.byref(n))
    if status not in (ZR_OK, ZR_ERANGE) or (status == ZR_ERANGE and n.value == 0):
        _check(status)
    buf = (_Fragment * max(1, n.value))()
    _check(_lib.zr_layout_fragments(layout.handle, int(begin), int(end), buf, n.value, ctypes.byref(n)))
    return [(f.tensor, f.tensor_offset, f.flat_offset, f.numel) for f in buf[:n.value]]


def zr_layout_ledger_bytes(layout: Layout, stage: int) -> int:
    out = ctypes.c_int64()
    _check(_lib.zr_layout_ledger_bytes(layout.handle, int(stage), ctypes.byref(out)))
    return out.value


# ----------------------------------------------------------- pack/unpack ----

ViewArg = Union[None, torch.Tensor, Tuple[torch.Tensor, int]]


def _views(layout: Layout, views: Sequence[ViewArg]):
    arr = (_View * max(1, len(views)))()
    for t, v in enumerate(views):
        if v is None:
            continue
        tensor, first = (v, 0) if isinstance(v, torch.Tensor) else v
        arr[t].ptr = _ptr(tensor, 2, f"views[{t}]")
        arr[t].first = int(first)
        arr[t].count = tensor.numel()
    return arr


def zr_pack(layout: Layout, views: Sequence[ViewArg], flat: torch.Tensor, begin: int, end: int,
            stream=None) -> None:
    """flat (holding flat elements [begin, end)) <- per-tensor views; padding zeroed.
    views[t] is None, a tensor holding all of tensor t, or (tensor, first)."""
    _need(int(end) - int(begin), flat=flat)
    _gpu_call(_lib.zr_pack, stream, (flat, views), layout.handle, _views(layout, views), len(views),
              _ptr(flat, 2, "flat"), int(begin), int(end))


def zr_unpack(layout: Layout, flat: torch.Tensor, begin: int, end: int, views: Sequence[ViewArg],
              stream=None) -> None:
    """per-tensor views <- flat elements [begin, end)."""
    _need(int(end) - int(begin), flat=flat)
    _gpu_call(_lib.zr_unpack, stream, (flat, views), layout.handle, _ptr(flat, 2, "flat"), int(begin), int(end),
              _views(layout, views), len(views))


# ------------------------------------------------------------ reduce/adamw ----

def zr_reduce_slice(contribs: Sequence[torch.Tensor], out: torch.Tensor, numel: Optional[int] = None,
                    stream=None) -> None:
    """out[i] = bf16(mean over k of contribs[k][i]) for i < numel (default out.numel())."""
    n = len(contribs)
    table = (ctypes.c_void_p * max(1, n))(*[_ptr(c, 2, f"contribs[{k}]") for k, c in enumerate(contribs)])
    numel = out.numel() if numel is None else int(numel)
    _need(numel, out=out, **{f"contribs[{k}]": c for k, c in enumerate(contribs)})
    _gpu_call(_lib.zr_reduce_slice, stream, (out, contribs), table, n, numel, _ptr(out, 2, "out"))


def zr_adamw_step(grad: torch.Tensor, master: torch.Tensor, exp_avg: torch.Tensor, exp_avg_sq: torch.Tensor,
                  param_out: Optional[torch.Tensor], *, lr: float, beta1: float, beta2: float, eps: float,
                  weight_decay: float, step: int, grad_scale: float = 1.0, numel: Optional[int] = None,
                  stream=None) -> None:
    """In-place AdamW on fp32 master/exp_avg/exp_avg_sq from a bf16 gradient, with
    the bf16 copy of the new master written to param_out (unless None)."""
    hp = _HParams(float(lr), float(beta1), float(beta2), float(eps), float(weight_decay), float(grad_scale),
                  int(step))
    numel = master.numel() if numel is None else int(numel)
    _need(numel, grad=grad, master=master, exp_avg=exp_avg, exp_avg_sq=exp_avg_sq, param_out=param_out)
    _gpu_call(_lib.zr_adamw_step, stream, (grad, master, exp_avg, exp_avg_sq, param_out), _ptr(grad, 2, "grad"),
              _ptr(master, 4, "master"), _ptr(exp_avg, 4, "exp_avg"), _ptr(exp_avg_sq, 4, "exp_avg_sq"),
              _ptr(param_out, 2, "param_out"), numel, ctypes.byref(hp))


def zr_reduce_adamw_step(contribs: Sequence[torch.Tensor], master: torch.Tensor, exp_avg: torch.Tensor,
                         exp_avg_sq: torch.Tensor, param_out: Optional[torch.Tensor],
                         grad_out: Optional[torch.Tensor] = None, *, lr: float, beta1: float, beta2: float,
                         eps: float, weight_decay: float, step: int, grad_scale: float = 1.0,
                         numel: Optional[int] = None, stream=None) -> None:
    """zr_reduce_slice(contribs -> mean) then zr_adamw_step(mean, ...) in one pass;
    grad_out (optional) receives the bf16 mean."""
    n = len(contribs)
    table = (ctypes.c_void_p * max(1, n))(*[_ptr(c, 2, f"contribs[{k}]") for k, c in enumerate(contribs)])
    hp = _HParams(float(lr), float(beta1), float(beta2), float(eps), float(weight_decay), float(grad_scale),
                  int(step))
    numel = master.numel() if numel is None else int(numel)
    _need(numel, master=master, exp_avg=exp_avg, exp_avg_sq=exp_avg_sq, param_out=param_out, grad_out=grad_out,
          **{f"contribs[{k}]": c for k, c in enumerate(contribs)})
    _gpu_call(_lib.zr_reduce_adamw_step, stream, (master, exp_avg, exp_avg_sq, param_out, grad_out, contribs),
              table, n, _ptr(master, 4, "master"), _ptr(exp_avg, 4, "exp_avg"), _ptr(exp_avg_sq, 4, "exp_avg_sq"),
              _ptr(param_out, 2, "param_out"), _ptr(grad_out, 2, "grad_out"), numel, ctypes.byref(hp))


# ------------------------------------------------------ fp16 + loss scale ----

def loss_scale_record(device=None) -> torch.Tensor:
    """A device tensor holding one zr_loss_scale record (16 bytes: float scale,
    int32 good_steps, int32 found_inf, int32 skipped), uninitialised."""
    return torch.empty(4, dtype=torch.int32, device=device if device is not None else "cuda")


def _ls(ls: Optional[torch.Tensor]) -> Optional[int]:
    if ls is None:
        return None
    p = _ptr(ls, 4, "ls")
    if ls.numel() < 4:
        raise ValueError("ls must hold at least 16 bytes")
    return p


def zr_loss_scale_init(ls: torch.Tensor, initial_scale: float = 2.0 ** 16, stream=None) -> None:
    _gpu_call(_lib.zr_loss_scale_init, stream, (ls,), _ls(ls), float(initial_scale))


def zr_reduce_slice_f16(contribs: Sequence[torch.Tensor], out: torch.Tensor, ls: Optional[torch.Tensor] = None,
                        numel: Optional[int] = None, stream=None) -> None:
    """out[i] = fp16(mean over k of contribs[k][i]); flags ls on inf or NaN."""
    n = len(contribs)
    table = (ctypes.c_void_p * max(1, n))(*[_ptr(c, 2, f"contribs[{k}]") for k, c in enumerate(contribs)])
    numel = out.numel() if numel is None else int(numel)
    _need(numel, out=out, **{f"contribs[{k}]": c for k, c in enumerate(contribs)})
    _gpu_call(_lib.zr_reduce_slice_f16, stream, (out, ls, contribs), table, n, numel, _ptr(out, 2, "out"), _ls(ls))


def zr_check_finite_f16(grad: torch.Tensor, ls: torch.Tensor, numel: Optional[int] = None, stream=None) -> None:
    numel = grad.numel() if numel is None else int(numel)
    _need(numel, grad=grad)
    _gpu_call(_lib.zr_check_finite_f16, stream, (grad, ls), _ptr(grad, 2, "grad"), numel, _ls(ls))


def zr_adamw_step_f16(grad: torch.Tensor, master: torch.Tensor, exp_avg: torch.Tensor, exp_avg_sq: torch.Tensor,
                      param_out: Optional[torch.Tensor], ls: torch.Tensor, *, lr: float, beta1: float, beta2: float,
                      eps: float, weight_decay: float, step: int, grad_scale: float = 1.0,
                      numel: Optional[int] = None, stream=None) -> None:
    """AdamW on the fp16 gradient divided by the loss scale; skipped while ls
    holds the overflow flag."""
    hp = _HParams(float(lr), float(beta1), float(beta2), float(eps), float(weight_decay), float(grad_scale),
                  int(step))
    numel = master.numel() if numel is None else int(numel)
    _need(numel, grad=grad, master=master, exp_avg=exp_avg, exp_avg_sq=exp_avg_sq, param_out=param_out)
    _gpu_call(_lib.zr_adamw_step_f16, stream, (grad, master, exp_avg, exp_avg_sq, param_out, ls),
              _ptr(grad, 2, "grad"), _ptr(master, 4, "master"), _ptr(exp_avg, 4, "exp_avg"),
              _ptr(exp_avg_sq, 4, "exp_avg_sq"), _ptr(param_out, 2, "param_out"), numel, ctypes.byref(hp), _ls(ls))


def zr_loss_scale_update(ls: torch.Tensor, window: int = 1000, factor: float = 2.0, min_scale: float = 1.0,
                         stream=None) -> None:
    _gpu_call(_lib.zr_loss_scale_update, stream, (ls,), _ls(ls), int(window), float(factor), float(min_scale))


# ---------------------------------------------------------- int8 gather ----

def _int8_sizes(numel: int, block: int, q: torch.Tensor, scales: torch.Tensor):
    if q.numel() < numel:
        raise ValueError(f"q holds {q.numel()} elements, {numel} needed")
    if block > 0 and scales.numel() < -(-numel // block):
        raise ValueError(f"scales holds {scales.numel()} entries, {-(-numel // block)} needed")


def zr_quantize_int8(src: torch.Tensor, q: torch.Tensor, scales: torch.Tensor, block: int = 2048,
                     numel: Optional[int] = None, stream=None) -> None:
    """Per block of `block` elements of bf16 src: scales[b] = amax / 127 and
    q[i] = rint(src[i] / scales[b]) clamped to +-127."""
    numel = src.numel() if numel is None else int(numel)
    _need(numel, src=src)
    _int8_sizes(numel, int(block), q, scales)
    _gpu_call(_lib.zr_quantize_int8, stream, (src, q, scales), _ptr(src, 2, "src"), numel, int(block),
              _ptr(q, 1, "q"), _ptr(scales, 4, "scales"))


def zr_dequantize_int8(q: torch.Tensor, scales: torch.Tensor, dst: torch.Tensor, block: int = 2048,
                       numel: Optional[int] = None, stream=None) -> None:
    """dst[i] = bf16(q[i] * scales[i // block])."""
    numel = dst.numel() if numel is None else int(numel)
    _need(numel, dst=dst)
    _int8_sizes(numel, int(block), q, scales)
    _gpu_call(_lib.zr_dequantize_int8, stream, (q, scales, dst), _ptr(q, 1, "q"), _ptr(scales, 4, "scales"), numel,
              int(block), _ptr(dst, 2, "dst"))


def zr_unpack_int8(layout: Layout, q: torch.Tensor, scales: torch.Tensor, begin: int, end: int,
                   views: Sequence[ViewArg], block: int = 2048, stream=None) -> None:
    """Per-tensor views <- bf16(code * scale) for flat elements [begin, end) of
    a quantized AllGather (per-shard blocks); q[k] is the code of element
    begin + k and scales[0] the scale of the block holding element begin."""
    _need(int(end) - int(begin), q=q)
    if end > begin and int(block) > 0:
        S = zr_layout_query(layout)["shard"]
        per_rank = -(-S // int(block))
        g = lambda i: (i // S) * per_rank + (i % S) // int(block)
        _need(g(int(end) - 1) - g(int(begin)) + 1, scales=scales)
    _gpu_call(_lib.zr_unpack_int8, stream, (q, scales, views), layout.handle, _ptr(q, 1, "q"),
              _ptr(scales, 4, "scales"), int(block), int(begin), int(end), _views(layout, views), len(views))


def _int4_sizes(numel: int, block: int, q4: torch.Tensor, scales: torch.Tensor):
    if q4.numel() * q4.element_size() < -(-numel // 2):
        raise ValueError(f"q4 holds {q4.numel() * q4.element_size()} bytes, {-(-numel // 2)} needed")
    if block > 0 and scales.numel() < -(-numel // block):
        raise ValueError(f"scales holds {scales.numel()} entries, {-(-numel // block)} needed")


def zr_quantize_int4(src: torch.Tensor, q4: torch.Tensor, scales: torch.Tensor, block: int = 2048,
                     numel: Optional[int] = None, stream=None) -> None:
    """As zr_quantize_int8 with 7 for 127; codes two per byte in q4 (uint8),
    element 2j in the low four bits of byte j."""
    numel = src.numel() if numel is None else int(numel)
    _need(numel, src=src)
    _int4_sizes(numel, int(block), q4, scales)
    _gpu_call(_lib.zr_quantize_int4, stream, (src, q4, scales), _ptr(src, 2, "src"), numel, int(block),
              _ptr(q4, 1, "q4"), _ptr(scales, 4, "scales"))


def zr_dequantize_int4(q4: torch.Tensor, scales: torch.Tensor, dst: torch.Tensor, block: int = 2048,
                       numel: Optional[int] = None, stream=None) -> None:
    """dst[i] = bf16(code i of q4 * scales[i // block])."""
    numel = dst.numel() if numel is None else int(numel)
    _need(numel, dst=dst)
    _int4_sizes(numel, int(block), q4, scales)
    _gpu_call(_lib.zr_dequantize_int4, stream, (q4, scales, dst), _ptr(q4, 1, "q4"), _ptr(scales, 4, "scales"), numel,
              int(block), _ptr(dst, 2, "dst"))


def zr_unpack_int4(layout: Layout, q4: torch.Tensor, scales: torch.Tensor, begin: int, end: int,
                   views: Sequence[ViewArg], block: int = 2048, stream=None) -> None:
    """Per-tensor views <- bf16(code * scale) for flat elements [begin, end) of
    an int4 quantized AllGather (codes and blocks per shard); q4[0] is the byte
    holding element begin's code and scales[0] the scale of its block."""
    if end > begin and int(block) > 0:
        S = zr_layout_query(layout)["shard"]
        per_rank, nbytes = -(-S // int(block)), -(-S // 2)
        g = lambda i: (i // S) * per_rank + (i % S) // int(block)
        cb = lambda i: (i // S) * nbytes + (i % S) // 2
        _need(g(int(end) - 1) - g(int(begin)) + 1, scales=scales)
        if q4.numel() * q4.element_size() < cb(int(end) - 1) - cb(int(begin)) + 1:
            raise ValueError("q4 is too short for the range")
    _gpu_call(_lib.zr_unpack_int4, stream, (q4, scales, views), layout.handle, _ptr(q4, 1, "q4"),
              _ptr(scales, 4, "scales"), int(block), int(begin), int(end), _views(layout, views), len(views))


# ------------------------------------------------------------ ZeRO-Offload ----

ZR_OFFLOAD_MIN_STAGING = 65536


def _on(t: Optional[torch.Tensor], kind: str, name: str):
    if t is not None and t.device.type != kind:
        raise ValueError(f"{name} must be a {kind} tensor")


def zr_host_simd() -> str:
    """Instruction set of the host AdamW: "avx512", "avx2" or "scalar"."""
    return _lib.zr_host_simd().decode()


def zr_host_adamw_step(grad: torch.Tensor, master: torch.Tensor, exp_avg: torch.Tensor, exp_avg_sq: torch.Tensor,
                       param_out: Optional[torch.Tensor], *, lr: float, beta1: float, beta2: float, eps: float,
                       weight_decay: float, step: int, grad_scale: float = 1.0, numel: Optional[int] = None,
                       threads: int = 0) -> None:
    """zr_adamw_step on host (CPU) tensors, on `threads` host threads (0: all)."""
    for t, name in ((grad, "grad"), (master, "master"), (exp_avg, "exp_avg"), (exp_avg_sq, "exp_avg_sq"),
                    (param_out, "param_out")):
        _on(t, "cpu", name)
    hp = _HParams(float(lr), float(beta1), float(beta2), float(eps), float(weight_decay), float(grad_scale),
                  int(step))
    numel = master.numel() if numel is None else int(numel)
    _need(numel, grad=grad, master=master, exp_avg=exp_avg, exp_avg_sq=exp_avg_sq, param_out=param_out)
    _check(_lib.zr_host_adamw_step(_ptr(grad, 2, "grad", "cpu"), _ptr(master, 4, "master", "cpu"),
                                   _ptr(exp_avg, 4, "exp_avg", "cpu"), _ptr(exp_avg_sq, 4, "exp_avg_sq", "cpu"),
                                   _ptr(param_out, 2, "param_out", "cpu"), numel, ctypes.byref(hp), int(threads)))


def offload_staging(nbytes: int = 64 << 20) -> torch.Tensor:
    """Pinned host staging buffer for zr_offload_adamw_step."""
    return torch.empty(int(nbytes), dtype=torch.uint8, pin_memory=True)


def zr_offload_adamw_step(grad: torch.Tensor, master: torch.Tensor, exp_avg: torch.Tensor, exp_avg_sq: torch.Tensor,
                          param_out: Optional[torch.Tensor], staging: torch.Tensor, *, lr: float, beta1: float,
                          beta2: float, eps: float, weight_decay: float, step: int, grad_scale: float = 1.0,
                          numel: Optional[int] = None, threads: int = 0, stream=None) -> None:
    """ZeRO-Offload step: device bf16 grad -> host AdamW on host fp32 master /
    exp_avg / exp_avg_sq -> device bf16 param_out, through the pinned staging
    buffer.  Returns when the parameters are on the device."""
    _on(grad, "cuda", "grad")
    _on(param_out, "cuda", "param_out")
    for t, name in ((master, "master"), (exp_avg, "exp_avg"), (exp_avg_sq, "exp_avg_sq"), (staging, "staging")):
        _on(t, "cpu", name)
    if not staging.is_pinned():
        raise ValueError("staging must be pinned host memory (see offload_staging)")
    hp = _HParams(float(lr), float(beta1), float(beta2), float(eps), float(weight_decay), float(grad_scale),
                  int(step))
    numel = master.numel() if numel is None else int(numel)
    _need(numel, grad=grad, master=master, exp_avg=exp_avg, exp_avg_sq=exp_avg_sq, param_out=param_out)
    _gpu_call(_lib.zr_offload_adamw_step, stream, (grad, param_out), _ptr(grad, 2, "grad"),
              _ptr(master, 4, "master", "cpu"), _ptr(exp_avg, 4, "exp_avg", "cpu"),
              _ptr(exp_avg_sq, 4, "exp_avg_sq", "cpu"), _ptr(param_out, 2, "param_out"), numel, ctypes.byref(hp),
              _ptr(staging, 1, "staging", "cpu"), staging.numel(), int(threads))


# ---------------------------------------------------------- captured steps ----

class Graph:
    """Owns a zr_graph (released on garbage collection)."""

    def __init__(self, handle: int):
        self._h = ctypes.c_void_p(handle)

    @property
    def handle(self):
        return self._h

    def __del__(self):
        if getattr(self, "_h", None) and self._h.value and _lib is not None:
            _lib.zr_graph_destroy(self._h)
            self._h = ctypes.c_void_p(None)


def zr_graph_capture_begin(stream=None) -> None:
    """Start recording library calls on `stream` (default: torch's current
    stream, which must not be the default stream)."""
    _check(_lib.zr_graph_capture_begin(_stream(stream)))


def zr_graph_capture_end(stream=None) -> Graph:
    h = ctypes.c_void_p()
    _check(_lib.zr_graph_capture_end(_stream(stream), ctypes.byref(h)))
    return Graph(h.value)


def zr_graph_info(g: Graph) -> Tuple[int, int]:
    """(kernel nodes, AdamW-family nodes) of a captured graph."""
    k, a = ctypes.c_int32(), ctypes.c_int32()
    _check(_lib.zr_graph_info(g.handle, ctypes.byref(k), ctypes.byref(a)))
    return k.value, a.value


def zr_graph_set_adamw(g: Graph, *, lr: float, beta1: float, beta2: float, eps: float, weight_decay: float,
                       step: int, grad_scale: float = 1.0) -> None:
    """AdamW hyper-parameters for the graph's following launches."""
    hp = _HParams(float(lr), float(beta1), float(beta2), float(eps), float(weight_decay), float(grad_scale),
                  int(step))
    _check(_lib.zr_graph_set_adamw(g.handle, ctypes.byref(hp)))


def zr_graph_launch(g: Graph, stream=None) -> None:
    _check(_lib.zr_graph_launch(g.handle, _stream(stream)))


def zr_graph_destroy(g: Graph) -> None:
    if g._h.value:
        _lib.zr_graph_destroy(g._h)
        g._h = ctypes.c_void_p(None)

