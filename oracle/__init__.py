"""Plain CPU oracle for one rank's share of a ZeRO-3 data-parallel step.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()`` and
the benchmark's ``cpu_baseline`` leg may import, call or execute anything in
this package.  It shares no code with the GPU library and imports nothing from
it; the two meet only at the seeded input generators of ``zr_workloads``.

What is here, each part written from the ZeRO-3 web pages:

* ``Layout``: the flat, padded, rank-contiguous partition with small-tensor
  persistence (pure Python integers, no vectorisation).
* ``ledger_closed_form`` / ``Layout.ledger_bytes``: per-rank model-state bytes.
* ``pack`` / ``unpack``: bit copies between per-tensor bf16 views and the flat
  buffer (numpy slice copies, one fragment at a time).
* ``reduce`` / ``adamw`` / bf16 conversion: scalar C loops in ``zr_oracle.c``
  (built by ``oracle/build.py`` with gcc, no fast-math, no FP contraction).

Parity pins for every function live in ``tests/test_oracle_*.py``; all of them
are pinned (none is "parity unpinned").
"""
from __future__ import annotations

import ctypes
import os
from fractions import Fraction
from typing import List, Optional, Sequence, Tuple

import numpy as np

from . import build as _build

DEFAULT_PERSIST_THRESHOLD = 100_000

_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIBRARY):
            _build.build()
        lib = ctypes.CDLL(_build.LIBRARY)
        i64, i32 = ctypes.c_int64, ctypes.c_int32
        p = ctypes.c_void_p
        d = ctypes.c_double
        lib.zr_oracle_bf16_from_f32.argtypes = [p, i64, p]
        lib.zr_oracle_bf16_from_f32.restype = None
        lib.zr_oracle_f32_from_bf16.argtypes = [p, i64, p]
        lib.zr_oracle_f32_from_bf16.restype = None
        lib.zr_oracle_reduce.argtypes = [p, i32, i64, p]
        lib.zr_oracle_reduce.restype = None
        lib.zr_oracle_adamw.argtypes = [p, p, p, p, p, i64, d, d, d, d, d, d, i64]
        lib.zr_oracle_adamw.restype = None
        lib.zr_oracle_f16_from_f32.argtypes = [p, i64, p]
        lib.zr_oracle_f16_from_f32.restype = None
        lib.zr_oracle_f32_from_f16.argtypes = [p, i64, p]
        lib.zr_oracle_f32_from_f16.restype = None
        lib.zr_oracle_reduce_f16.argtypes = [p, i32, i64, p]
        lib.zr_oracle_reduce_f16.restype = None
        lib.zr_oracle_found_inf_f16.argtypes = [p, i64]
        lib.zr_oracle_found_inf_f16.restype = i32
        lib.zr_oracle_adamw_f16.argtypes = [p, p, p, p, p, i64, d, d, d, d, d, d, i64, d]
        lib.zr_oracle_adamw_f16.restype = None
        lib.zr_oracle_quantize_int8.argtypes = [p, i64, i32, p, p]
        lib.zr_oracle_quantize_int8.restype = None
        lib.zr_oracle_dequantize_int8.argtypes = [p, p, i64, i32, p]
        lib.zr_oracle_dequantize_int8.restype = None
        lib.zr_oracle_quantize_int4.argtypes = [p, i64, i32, p, p]
        lib.zr_oracle_quantize_int4.restype = None
        lib.zr_oracle_dequantize_int4.argtypes = [p, p, i64, i32, p]
        lib.zr_oracle_dequantize_int4.restype = None
        _lib = lib
    return _lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _check(a: np.ndarray, dtype, name: str):
    if not isinstance(a, np.ndarray) or a.dtype != dtype or not a.flags["C_CONTIGUOUS"]:
        raise TypeError(f"{name} must be a C-contiguous numpy array of {np.dtype(dtype).name}")


# ------------------------------------------------------------------ bf16 ----

def bf16_from_f32(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bits, round to nearest even; NaN stays NaN.

    The concept page's Stage 1 mechanism converts the updated fp32 master to the
    16-bit working copy; the ledger section of the ddp-to-zero blog makes that
    copy bf16.  Round-to-nearest-even is the reading taken for the conversion.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    _load().zr_oracle_bf16_from_f32(_ptr(x), x.size, _ptr(out))
    return out


def f32_from_bf16(h: np.ndarray) -> np.ndarray:
    """bf16 bits -> fp32 (exact widening)."""
    h = np.ascontiguousarray(h, dtype=np.uint16)
    out = np.empty(h.shape, dtype=np.float32)
    _load().zr_oracle_f32_from_bf16(_ptr(h), h.size, _ptr(out))
    return out


# ---------------------------------------------------------------- reduce ----

def reduce(contribs: Sequence[np.ndarray], out: Optional[np.ndarray] = None) -> np.ndarray:
    """Mean of n bf16 gradient contributions, element by element (bf16 bits in,
    bf16 bits out), accumulated in fp32 in ascending contribution order.

    Follows the ddp-to-zero blog, "ZeRO-2: why gradients can be sharded" (the
    averaged-gradient ReduceScatter worked example).  ``out`` may be
    ``contribs[0]`` itself.
    """
    if len(contribs) < 1:
        raise ValueError("need at least one contribution")
    numel = contribs[0].size
    for k, c in enumerate(contribs):
        _check(c, np.uint16, f"contribs[{k}]")
        if c.size != numel:
            raise ValueError("contributions differ in length")
    if out is None:
        out = np.empty(numel, dtype=np.uint16)
    _check(out, np.uint16, "out")
    if out.size != numel:
        raise ValueError("out has the wrong length")
    table = (ctypes.c_void_p * len(contribs))(*[_ptr(c) for c in contribs])
    _load().zr_oracle_reduce(ctypes.cast(table, ctypes.c_void_p), len(contribs), numel, _ptr(out))
    return out


# ----------------------------------------------------------------- AdamW ----

def adamw(grad: np.ndarray, master: np.ndarray, exp_avg: np.ndarray, exp_avg_sq: np.ndarray,
          param_out: Optional[np.ndarray], *, lr: float, beta1: float, beta2: float, eps: float,
          weight_decay: float, step: int, grad_scale: float = 1.0) -> None:
    """One AdamW step in place on fp32 master / exp_avg / exp_avg_sq from a bf16
    gradient, then the bf16 copy of the new master into ``param_out`` (if given).

    Computed in double, stored in the pages' dtypes (fp32 states, bf16 copy).
    Follows the ddp-to-zero blog's ledger section and "ZeRO-1: why optimizer
    states can be sharded", the concept page's Stage 1 mechanism, and the
    tutorial's section 3.1 AdamW configuration; the formula is the published
    decoupled-weight-decay Adam (see zr_oracle.c).
    """
    n = grad.size
    _check(grad, np.uint16, "grad")
    for name, a in (("master", master), ("exp_avg", exp_avg), ("exp_avg_sq", exp_avg_sq)):
        _check(a, np.float32, name)
        if a.size != n:
            raise ValueError(f"{name} has the wrong length")
    pp = None
    if param_out is not None:
        _check(param_out, np.uint16, "param_out")
        if param_out.size != n:
            raise ValueError("param_out has the wrong length")
        pp = _ptr(param_out)
    if step < 1:
        raise ValueError("step must be >= 1")
    _load().zr_oracle_adamw(_ptr(grad), _ptr(master), _ptr(exp_avg), _ptr(exp_avg_sq), pp, n,
                            float(lr), float(beta1), float(beta2), float(eps),
                            float(weight_decay), float(grad_scale), int(step))


# ------------------------------------------------------------------ fp16 ----
#
# fp16 parameters and gradients with dynamic loss scaling: the ZeRO tutorial
# (cnhsyj.com) 3.1 sets fp16 with a dynamic loss scale (loss_scale 0), window
# 1000 and initial scale 2^16, and 4.2 recommends dynamic scaling for fp16
# gradients that are very small or very large; the concept page
# (compassingai.com) 16 B/param table uses fp16 parameters and gradients.

def f16_from_f32(x: np.ndarray) -> np.ndarray:
    """fp32 -> fp16 bits, round to nearest even; overflow to inf; NaN to the
    quiet NaN 0x7e00 with the input's sign."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    _load().zr_oracle_f16_from_f32(_ptr(x), x.size, _ptr(out))
    return out


def f32_from_f16(h: np.ndarray) -> np.ndarray:
    """fp16 bits -> fp32 (exact)."""
    h = np.ascontiguousarray(h, dtype=np.uint16)
    out = np.empty(h.shape, dtype=np.float32)
    _load().zr_oracle_f32_from_f16(_ptr(h), h.size, _ptr(out))
    return out


def reduce_f16(contribs: Sequence[np.ndarray], out: Optional[np.ndarray] = None) -> np.ndarray:
    """Mean of n fp16 contributions (fp32 sum in ascending k, one division, fp16)."""
    numel = contribs[0].size
    for k, c in enumerate(contribs):
        _check(c, np.uint16, f"contribs[{k}]")
        if c.size != numel:
            raise ValueError("contributions differ in length")
    if out is None:
        out = np.empty(numel, dtype=np.uint16)
    table = (ctypes.c_void_p * len(contribs))(*[_ptr(c) for c in contribs])
    _load().zr_oracle_reduce_f16(ctypes.cast(table, ctypes.c_void_p), len(contribs), numel, _ptr(out))
    return out


def found_inf_f16(x: np.ndarray) -> bool:
    """True if any fp16 value is inf or NaN."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    return bool(_load().zr_oracle_found_inf_f16(_ptr(x), x.size))


def adamw_f16(grad: np.ndarray, master: np.ndarray, exp_avg: np.ndarray, exp_avg_sq: np.ndarray,
              param_out: Optional[np.ndarray], *, lr: float, beta1: float, beta2: float, eps: float,
              weight_decay: float, step: int, loss_scale: float, grad_scale: float = 1.0) -> None:
    """The AdamW step of ``adamw`` on an fp16 gradient that carries the loss
    scale (divided out before the update), with an fp16 copy."""
    n = grad.size
    _check(grad, np.uint16, "grad")
    for name, a in (("master", master), ("exp_avg", exp_avg), ("exp_avg_sq", exp_avg_sq)):
        _check(a, np.float32, name)
        if a.size != n:
            raise ValueError(f"{name} has the wrong length")
    pp = None
    if param_out is not None:
        _check(param_out, np.uint16, "param_out")
        pp = _ptr(param_out)
    _load().zr_oracle_adamw_f16(_ptr(grad), _ptr(master), _ptr(exp_avg), _ptr(exp_avg_sq), pp, n,
                                float(lr), float(beta1), float(beta2), float(eps), float(weight_decay),
                                float(grad_scale), int(step), float(loss_scale))


class LossScale:
    """Dynamic loss scale, the plain rule: a step whose gradient holds an inf or
    NaN is skipped and the scale is divided by ``factor`` (not below
    ``min_scale``); after ``window`` consecutive clean steps the scale is
    multiplied by ``factor``.  Defaults follow the tutorial's fp16 config
    (initial scale 2^16, window 1000); the factor 2 and the floor 1 are the
    customary values the page leaves implicit."""

    def __init__(self, initial: float = 2.0 ** 16, window: int = 1000, factor: float = 2.0,
                 min_scale: float = 1.0):
        self.scale = float(initial)
        self.window = int(window)
        self.factor = float(factor)
        self.min_scale = float(min_scale)
        self.good_steps = 0
        self.skipped = 0

    def update(self, found_inf: bool) -> None:
        if found_inf:
            self.scale = max(self.scale / self.factor, self.min_scale)
            self.good_steps = 0
            self.skipped += 1
        else:
            self.good_steps += 1
            if self.good_steps == self.window:
                self.scale = self.scale * self.factor
                self.good_steps = 0


def step_f16(contribs: Sequence[np.ndarray], master: np.ndarray, exp_avg: np.ndarray, exp_avg_sq: np.ndarray,
             param_out: Optional[np.ndarray], scaler: LossScale, *, lr: float, beta1: float, beta2: float,
             eps: float, weight_decay: float, step: int, grad_scale: float = 1.0) -> np.ndarray:
    """One fp16 step with dynamic loss scaling: the mean of the scaled fp16
    contributions; if it holds an inf or NaN the update is skipped (state and
    copy untouched), else AdamW on the unscaled mean; then the scale update.
    Returns the fp16 mean."""
    grad = reduce_f16(contribs)
    inf = found_inf_f16(grad)
    if not inf:
        adamw_f16(grad, master, exp_avg, exp_avg_sq, param_out, lr=lr, beta1=beta1, beta2=beta2, eps=eps,
                  weight_decay=weight_decay, step=step, loss_scale=scaler.scale, grad_scale=grad_scale)
    scaler.update(inf)
    return grad


# ------------------------------------------------------------------ int8 ----

def quantize_int8(src: np.ndarray, block: int) -> Tuple[np.ndarray, np.ndarray]:
    """Symmetric block-wise int8 quantization of bf16 bits (the weights of the
    quantized AllGather, ZeRO++ qwZ on the concept page (compassingai.com)):
    per block s = amax / 127, q = rint(x / s) clamped to +-127.  Returns
    (q int8 [numel], scales fp32 [ceil(numel / block)])."""
    _check(src, np.uint16, "src")
    if block < 1:
        raise ValueError("block must be >= 1")
    q = np.empty(src.size, dtype=np.int8)
    scales = np.empty(-(-src.size // block), dtype=np.float32)
    _load().zr_oracle_quantize_int8(_ptr(src), src.size, int(block), _ptr(q), _ptr(scales))
    return q, scales


def dequantize_int8(q: np.ndarray, scales: np.ndarray, block: int) -> np.ndarray:
    """bf16 bits of q * s, rounded to nearest even."""
    _check(q, np.int8, "q")
    _check(scales, np.float32, "scales")
    if scales.size != -(-q.size // block):
        raise ValueError("scales has the wrong length")
    out = np.empty(q.size, dtype=np.uint16)
    _load().zr_oracle_dequantize_int8(_ptr(q), _ptr(scales), q.size, int(block), _ptr(out))
    return out


def quantize_int4(src: np.ndarray, block: int) -> Tuple[np.ndarray, np.ndarray]:
    """Symmetric block-wise int4 quantization of bf16 bits (ZeRO++ qwZ names
    int4 beside int8 on the concept page (compassingai.com); the int8 rule with
    7 for 127): per block s = amax / 7, q = rint(x / s) clamped to +-7; two
    codes per byte, element 2j in the low four bits of byte j.  Returns
    (q4 uint8 [ceil(numel / 2)], scales fp32 [ceil(numel / block)])."""
    _check(src, np.uint16, "src")
    if block < 1:
        raise ValueError("block must be >= 1")
    q4 = np.empty(-(-src.size // 2), dtype=np.uint8)
    scales = np.empty(-(-src.size // block), dtype=np.float32)
    _load().zr_oracle_quantize_int4(_ptr(src), src.size, int(block), _ptr(q4), _ptr(scales))
    return q4, scales


def dequantize_int4(q4: np.ndarray, scales: np.ndarray, numel: int, block: int) -> np.ndarray:
    """bf16 bits of q * s for the first numel codes of q4, rounded to nearest even."""
    _check(q4, np.uint8, "q4")
    _check(scales, np.float32, "scales")
    if q4.size < -(-numel // 2) or scales.size != -(-numel // block):
        raise ValueError("q4 or scales has the wrong length")
    out = np.empty(numel, dtype=np.uint16)
    _load().zr_oracle_dequantize_int4(_ptr(q4), _ptr(scales), numel, int(block), _ptr(out))
    return out


# ---------------------------------------------------------------- layout ----

class Layout:
    """Flat, padded partition of a tensor list over ``n_d`` data-parallel ranks.

    Rules, each from the pages:

    * A tensor with fewer than ``threshold`` elements is persistent: it is not
      partitioned and stays whole on every rank (Zero-3 parameter-partitioning
      article (hotelren.com): the quick-start config's
      stage3_param_persistence_threshold of 100000, and the small-parameter
      residency paragraph; "below" is read as strictly less than).
    * The other tensors are concatenated in list order into one flat buffer
      with no gaps between tensors (tutorial section 3.2, contiguous_gradients).
    * The flat buffer is split into ``n_d`` equal contiguous slices in rank
      order: rank 0 owns the first slice, rank 1 the next (tutorial section 2.1;
      the ddp-to-zero blog's 8-parameter example in "ZeRO-3: why parameters can
      be sharded", where rank r holds elements 2r and 2r+1).
    * The pages assume n_d divides the element count; where it does not, the
      buffer is padded with zeros at its end up to the next multiple of n_d.
    * Persistent tensors are laid out one after another, in list order, in a
      separate replicated region.
    """

    def __init__(self, numels: Sequence[int], n_d: int, threshold: int = DEFAULT_PERSIST_THRESHOLD):
        numels = [int(x) for x in numels]
        if n_d < 1:
            raise ValueError("n_d must be >= 1")
        if threshold < 0:
            raise ValueError("threshold must be >= 0")
        if any(x < 0 for x in numels):
            raise ValueError("negative numel")
        self.numels = numels
        self.n_d = int(n_d)
        self.threshold = int(threshold)
        self.persistent = [x < self.threshold for x in numels]
        self.offset: List[int] = []
        flat = 0
        persist = 0
        for x, is_persistent in zip(numels, self.persistent):
            if is_persistent:
                self.offset.append(persist)
                persist += x
            else:
                self.offset.append(flat)
                flat += x
        self.psi = sum(numels)
        self.psi_part = flat
        self.psi_persist = persist
        # smallest multiple of n_d that is >= psi_part
        self.psi_pad = -(-self.psi_part // self.n_d) * self.n_d
        self.shard = self.psi_pad // self.n_d
        self.n_partitioned = sum(1 for q in self.persistent if not q)
        self.n_persistent = len(numels) - self.n_partitioned

    def rank_range(self, rank: int) -> Tuple[int, int]:
        """Flat elements [begin, end) owned by ``rank``."""
        if not 0 <= rank < self.n_d:
            raise IndexError("rank out of range")
        return rank * self.shard, (rank + 1) * self.shard

    def owner(self, j: int) -> int:
        """Rank owning flat element j (0 <= j < psi_pad)."""
        return j // self.shard

    def fragments(self, begin: int, end: int) -> List[Tuple[int, int, int, int]]:
        """Pieces of partitioned tensors inside flat [begin, end), in flat order,
        as (tensor, offset inside the tensor, flat offset, element count)."""
        if not 0 <= begin <= end <= self.psi_pad:
            raise ValueError("range outside [0, psi_pad]")
        out = []
        for t, x in enumerate(self.numels):
            if self.persistent[t] or x == 0:
                continue
            lo = max(begin, self.offset[t])
            hi = min(end, self.offset[t] + x)
            if lo < hi:
                out.append((t, lo - self.offset[t], lo, hi - lo))
        return out

    def ledger_bytes(self, stage: int) -> int:
        """Exact per-rank model-state bytes for this layout (16 B per element as
        2 bf16 param + 2 bf16 grad + 12 fp32 master/m/v).  Persistent tensors
        keep all of their state on every rank; partitioned state is one shard
        of ``shard`` elements (padding included)."""
        owned = self.shard + self.psi_persist
        if stage == 0:
            return 16 * self.psi
        if stage == 1:
            return 2 * self.psi + 2 * self.psi + 12 * owned
        if stage == 2:
            return 2 * self.psi + 14 * owned
        if stage == 3:
            return 16 * owned
        raise ValueError("stage must be 0..3")


def ledger_closed_form(psi: int, n_d: int, stage: int) -> Fraction:
    """Per-rank model-state bytes from the pages' closed forms (mixed precision
    with Adam: 16 bytes per parameter).

    Stage 0 (plain data parallel) 16 psi; stage 1 4 psi + 12 psi / n_d;
    stage 2 2 psi + 14 psi / n_d; stage 3 16 psi / n_d = (2+2+12) psi / n_d.
    Follows the concept page's per-stage memory formulas and their summary
    table, and the encyclopedia entry's principle section ((2+2+K) psi / N_d
    with K = 12 for Adam).
    """
    psi = Fraction(psi)
    if stage == 0:
        return 16 * psi
    if stage == 1:
        return 4 * psi + 12 * psi / n_d
    if stage == 2:
        return 2 * psi + 14 * psi / n_d
    if stage == 3:
        return (2 + 2 + 12) * psi / n_d
    raise ValueError("stage must be 0..3")


# ----------------------------------------------------------- pack/unpack ----

View = Optional[Tuple[np.ndarray, int]]  # (bf16 bits of elements [first, first+len), first)


def pack(layout: Layout, views: Sequence[View], begin: int, end: int) -> np.ndarray:
    """Flat bf16 elements [begin, end) gathered from per-tensor views; padding
    and anything outside the tensors is zero.  Bit copy.

    This is the local side of the AllGather / contiguous buffer: the ddp-to-zero
    blog's ZeRO-1 example reassembles [9] and [18] into [9, 18]; the tutorial's
    section 3.2 keeps gradients in one contiguous buffer.
    """
    flat = np.zeros(end - begin, dtype=np.uint16)
    for t, toff, foff, n in layout.fragments(begin, end):
        arr, first = views[t]
        flat[foff - begin: foff - begin + n] = arr[toff - first: toff - first + n]
    return flat


def unpack(layout: Layout, flat: np.ndarray, begin: int, end: int, views: Sequence[View]) -> None:
    """Scatter flat bf16 elements [begin, end) back into the per-tensor views
    (in place); the padding is not written anywhere.  Bit copy."""
    for t, toff, foff, n in layout.fragments(begin, end):
        arr, first = views[t]
        arr[toff - first: toff - first + n] = flat[foff - begin: foff - begin + n]


# ------------------------------------------------- quantized weight gather ----

def quantize_gathered(layout: Layout, flat: np.ndarray, block: int) -> Tuple[np.ndarray, np.ndarray]:
    """The quantized AllGather of the whole flat buffer (bf16 bits of
    [0, psi_pad)): every rank r quantizes its own shard flat[r S, (r+1) S) by
    quantize_int8 -- blocks start afresh at every shard, and a shard's last
    block is short when the block size does not divide S -- and the gather
    concatenates codes and scales in rank order (ceil(S / block) scales per
    rank).  ZeRO++ qwZ on the concept page (compassingai.com): the weights
    cross the AllGather quantized."""
    _check(flat, np.uint16, "flat")
    if flat.size != layout.psi_pad:
        raise ValueError("flat must hold psi_pad elements")
    S = layout.shard
    codes, scales = [], []
    for r in range(layout.n_d):
        q, s = quantize_int8(np.ascontiguousarray(flat[r * S:(r + 1) * S]), block)
        codes.append(q)
        scales.append(s)
    return np.concatenate(codes), np.concatenate(scales)


def gathered_block(layout: Layout, i: np.ndarray, block: int) -> np.ndarray:
    """Index into the gathered scales of the block that holds flat element i:
    rank r = i // S, then block (i - r S) // block of that rank's shard."""
    S = layout.shard
    per_rank = -(-S // block)
    r = i // S
    return r * per_rank + (i - r * S) // block


def unpack_int8(layout: Layout, q: np.ndarray, scales: np.ndarray, block: int, begin: int, end: int,
                views: Sequence[View]) -> None:
    """Receiver side of the quantized AllGather: flat elements [begin, end) are
    rebuilt as bf16(code * scale of their block) and scattered into the views
    like unpack.  q[k] is the code of flat element begin + k; scales[0] is the
    scale of the block holding element begin, and the rest follow in gathered
    order."""
    _check(q, np.int8, "q")
    _check(scales, np.float32, "scales")
    if end <= begin:
        return
    i = np.arange(begin, end, dtype=np.int64)
    g = gathered_block(layout, i, block)
    x = q[: end - begin].astype(np.float32) * scales[g - g[0]]
    unpack(layout, bf16_from_f32(x), begin, end, views)


def quantize_gathered_int4(layout: Layout, flat: np.ndarray, block: int) -> Tuple[np.ndarray, np.ndarray]:
    """The int4 quantized AllGather of the whole flat buffer: every rank r runs
    quantize_int4 on its own shard flat[r S, (r+1) S) -- blocks and the packing
    start afresh at every shard, ceil(S / 2) bytes and ceil(S / block) scales
    per rank -- and the gather concatenates codes and scales in rank order."""
    _check(flat, np.uint16, "flat")
    if flat.size != layout.psi_pad:
        raise ValueError("flat must hold psi_pad elements")
    S = layout.shard
    codes, scales = [], []
    for r in range(layout.n_d):
        q, s = quantize_int4(np.ascontiguousarray(flat[r * S:(r + 1) * S]), block)
        codes.append(q)
        scales.append(s)
    return np.concatenate(codes), np.concatenate(scales)


def gathered_code_byte(layout: Layout, i: np.ndarray) -> np.ndarray:
    """Byte of the int4 gathered codes holding flat element i's code: rank
    r = i // S, then byte (i - r S) // 2 of that rank's ceil(S / 2); the code is
    in the high four bits when (i - r S) is odd."""
    S = layout.shard
    r = i // S
    return r * (-(-S // 2)) + (i - r * S) // 2


def unpack_int4(layout: Layout, q4: np.ndarray, scales: np.ndarray, block: int, begin: int, end: int,
                views: Sequence[View]) -> None:
    """Receiver side of the int4 quantized AllGather: flat elements [begin,
    end) rebuilt as bf16(code * scale of their block) and scattered into the
    views like unpack.  q4[0] is the byte holding element begin's code and
    scales[0] the scale of the block holding element begin; the rest follow in
    gathered order."""
    _check(q4, np.uint8, "q4")
    _check(scales, np.float32, "scales")
    if end <= begin:
        return
    S = layout.shard
    i = np.arange(begin, end, dtype=np.int64)
    byte = gathered_code_byte(layout, i)
    high = ((i - (i // S) * S) % 2).astype(np.uint8)
    nibble = (q4[byte - byte[0]] >> (4 * high)) & 0xF
    code = nibble.astype(np.int16) - 16 * (nibble >= 8)
    g = gathered_block(layout, i, block)
    x = code.astype(np.float32) * scales[g - g[0]]
    unpack(layout, bf16_from_f32(x), begin, end, views)
