"""Seeded synthetic inputs (torch generators), shared by the oracle tests, the
GPU tests and the benchmark.  Holds none of the method's arithmetic: only
random numbers of the stated distributions, rounded to the stated dtypes.

A given (seed, device, size) always yields the same bits.  CPU and GPU
generators yield different streams, so tests that compare both sides generate
once and copy.
"""
from __future__ import annotations

from typing import Dict, List

import torch

from .configs import Workload

CHUNK = 1 << 28  # elements generated per generator call (bounds temporaries)

# array ids mixed into the seed
MASTER, EXP_AVG, EXP_AVG_SQ, GRAD, BITS = 1, 2, 3, 4, 5


def seed_of(base: int, array: int, step: int = 0, k: int = 0) -> int:
    return ((base * 1_000_003 + array) * 10_007 + step) * 1_009 + k


def _fill(out: torch.Tensor, seed: int, draw) -> torch.Tensor:
    g = torch.Generator(device=out.device)
    g.manual_seed(seed)
    n = out.numel()
    for s in range(0, n, CHUNK):
        e = min(n, s + CHUNK)
        out[s:e].copy_(draw(e - s, g))
    return out


def normal_f32(numel: int, std: float, seed: int, device="cpu") -> torch.Tensor:
    out = torch.empty(numel, dtype=torch.float32, device=device)
    if std == 0.0:
        return out.zero_()
    return _fill(out, seed, lambda n, g: torch.randn(n, generator=g, device=device) * std)


def uniform_f32(numel: int, high: float, seed: int, device="cpu") -> torch.Tensor:
    out = torch.empty(numel, dtype=torch.float32, device=device)
    if high == 0.0:
        return out.zero_()
    return _fill(out, seed, lambda n, g: torch.rand(n, generator=g, device=device) * high)


def normal_bf16(numel: int, std: float, seed: int, device="cpu") -> torch.Tensor:
    """N(0, std) draws rounded to bf16 (returned as torch.bfloat16)."""
    out = torch.empty(numel, dtype=torch.bfloat16, device=device)
    return _fill(out, seed,
                 lambda n, g: (torch.randn(n, generator=g, device=device) * std).to(torch.bfloat16))


def random_bits16(numel: int, seed: int, device="cpu") -> torch.Tensor:
    """Uniformly random 16-bit patterns (NaN payloads, -0, subnormals included),
    returned as torch.int16 so no arithmetic ever touches them."""
    out = torch.empty(numel, dtype=torch.int16, device=device)
    return _fill(out, seed, lambda n, g: torch.randint(-32768, 32768, (n,), generator=g,
                                                       device=device, dtype=torch.int16))


def shard_state(w: Workload, numel: int, device="cpu", salt: int = 0) -> Dict[str, torch.Tensor]:
    """fp32 master / exp_avg / exp_avg_sq of ``numel`` elements for workload w."""
    base = w.seed + salt
    return dict(
        master=normal_f32(numel, w.master_std, seed_of(base, MASTER), device),
        exp_avg=normal_f32(numel, w.m_std, seed_of(base, EXP_AVG), device),
        exp_avg_sq=uniform_f32(numel, w.v_high, seed_of(base, EXP_AVG_SQ), device),
    )


def contributions(w: Workload, numel: int, step_index: int = 0, device="cpu",
                  salt: int = 0) -> List[torch.Tensor]:
    """The n simulated per-rank bf16 gradient contributions for one step."""
    base = w.seed + salt
    return [normal_bf16(numel, w.grad_std, seed_of(base, GRAD, step_index, k), device)
            for k in range(w.n_contrib)]
