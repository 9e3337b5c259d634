"""Helpers for the GPU parity tests: device placement at chosen element
offsets inside guarded allocations, bit views, and the parity tolerances.

Parity tolerances:
* indexing, layout, pack/unpack, reduce: bit-exact;
* fp32 master / m / v: |gpu - ref| <= 1e-6 |ref| + 1e-9;
* bf16 parameter copy: within 1 bf16 ulp (order-mapped integers, +0 == -0).
The AdamW kernels compute the oracle's double update in the same order and
round each state once, so their outputs are also checked bit for bit
(assert_*_exact: the bar first, for a readable failure, then every bit).
"""
import sys

import numpy as np
import pytest
import torch

GUARD = 64
GUARD_U16 = 0x5A5A
GUARD_F32_BITS = 0x7FBADBAD  # a NaN pattern nobody computes
GUARD_I8 = -128  # outside the int8 code range [-127, 127]
GUARD_U8 = 0x88  # two int4 codes of -8, outside the int4 code range [-7, 7]


def device():
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a visible GPU")
    return torch.device("cuda:0")


def say(*args):
    print("[gpu-test]", *args, file=sys.stderr, flush=True)


def u16(t: torch.Tensor) -> np.ndarray:
    """Bits of a 2-byte tensor as numpy uint16."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def f32(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().cpu().numpy().astype(np.float32, copy=False)


class Placed:
    """A device copy of `host` at element `offset` inside a guarded allocation."""

    def __init__(self, host: np.ndarray, offset: int = 0, dev=None):
        dev = dev or device()
        n = host.size
        if host.dtype == np.uint16:
            big = torch.full((offset + n + GUARD,), GUARD_U16, dtype=torch.int16)
            big[offset:offset + n] = torch.from_numpy(host.view(np.int16).copy())
            self.guard_bits = np.uint16(GUARD_U16)
        elif host.dtype == np.float32:
            big = torch.from_numpy(np.full(offset + n + GUARD, GUARD_F32_BITS, dtype=np.uint32).view(np.float32))
            big[offset:offset + n] = torch.from_numpy(host.copy())
            self.guard_bits = np.uint32(GUARD_F32_BITS)
        elif host.dtype == np.int8:
            big = torch.full((offset + n + GUARD,), GUARD_I8, dtype=torch.int8)
            big[offset:offset + n] = torch.from_numpy(host.copy())
            self.guard_bits = np.int8(GUARD_I8)
        elif host.dtype == np.uint8:
            big = torch.full((offset + n + GUARD,), GUARD_U8, dtype=torch.uint8)
            big[offset:offset + n] = torch.from_numpy(host.copy())
            self.guard_bits = np.uint8(GUARD_U8)
        else:
            raise TypeError(host.dtype)
        self.big = big.to(dev)
        self.offset, self.n = offset, n
        self.view = self.big[offset:offset + n]

    def host(self) -> np.ndarray:
        if self.view.dtype == torch.int16:
            return u16(self.view)
        if self.view.dtype in (torch.int8, torch.uint8):
            return self.view.cpu().numpy().copy()
        return f32(self.view)

    def guards_intact(self) -> bool:
        b = self.big.cpu().numpy()
        if b.dtype not in (np.int8, np.uint8):
            b = b.view(np.uint16) if b.dtype == np.int16 else b.view(np.uint32)
        return bool(np.all(b[:self.offset] == self.guard_bits) and np.all(b[self.offset + self.n:] == self.guard_bits))


def assert_fp32_close(got: np.ndarray, ref: np.ndarray, what: str):
    g = got.astype(np.float64)
    r = ref.astype(np.float64)
    bad = ~(np.abs(g - r) <= 1e-6 * np.abs(r) + 1e-9)
    if bad.any():
        i = int(np.flatnonzero(bad)[0])
        raise AssertionError(f"{what}: {int(bad.sum())} of {got.size} outside 1e-6 rel + 1e-9 abs; "
                             f"first at {i}: gpu {got[i]!r} oracle {ref[i]!r}")


def bf16_order(h: np.ndarray) -> np.ndarray:
    h = h.astype(np.int64)
    return np.where(h & 0x8000, -(h & 0x7FFF), h)


def assert_bf16_within_1ulp(got: np.ndarray, ref: np.ndarray, what: str):
    d = np.abs(bf16_order(got) - bf16_order(ref))
    if (d > 1).any():
        i = int(np.flatnonzero(d > 1)[0])
        raise AssertionError(f"{what}: {int((d > 1).sum())} elements beyond 1 bf16 ulp; first at {i}: "
                             f"gpu {got[i]:#06x} oracle {ref[i]:#06x}")


def assert_bits_equal(got: np.ndarray, ref: np.ndarray, what: str):
    if got.shape != ref.shape:
        raise AssertionError(f"{what}: shape {got.shape} vs {ref.shape}")
    if got.size == 0:
        return
    ne = got.view(np.uint8).reshape(got.size, -1) != ref.view(np.uint8).reshape(ref.size, -1)
    ne = ne.any(axis=1)
    if ne.any():
        i = int(np.flatnonzero(ne)[0])
        raise AssertionError(f"{what}: {int(ne.sum())} of {got.size} differ; first at {i}: "
                             f"gpu {got[i]!r} oracle {ref[i]!r}")


def assert_bf16_equal_nan_as_class(got: np.ndarray, ref: np.ndarray, what: str):
    """bf16 bit patterns: every element whose oracle value is a NaN must be a
    NaN, every other element must have the oracle's bits.  A NaN's sign and
    payload follow the arithmetic unit that made it (an x86 host gives 0 * inf
    a negative NaN, the GPU a positive one), so they are not compared."""
    g = np.ascontiguousarray(got, np.uint16)
    r = np.ascontiguousarray(ref, np.uint16)
    if g.shape != r.shape:
        raise AssertionError(f"{what}: shape {g.shape} vs {r.shape}")
    rn = (r & 0x7FFF) > 0x7F80
    gn = (g & 0x7FFF) > 0x7F80
    if (rn & ~gn).any():
        i = int(np.flatnonzero(rn & ~gn)[0])
        raise AssertionError(f"{what}: {int((rn & ~gn).sum())} oracle NaNs not NaN; first at {i}: gpu {g[i]:#06x}")
    assert_bits_equal(g[~rn], r[~rn], what + " (non-NaN values)")


def assert_fp32_exact(got: np.ndarray, ref: np.ndarray, what: str):
    assert_fp32_close(got, ref, what)
    assert_bits_equal(np.ascontiguousarray(got, np.float32), np.ascontiguousarray(ref, np.float32), f"{what} (bits)")


def assert_bf16_exact(got: np.ndarray, ref: np.ndarray, what: str):
    assert_bf16_within_1ulp(got, ref, what)
    assert_bits_equal(np.ascontiguousarray(got, np.uint16), np.ascontiguousarray(ref, np.uint16), f"{what} (bits)")
