"""Every rank's share of one data-parallel step, run one rank after another on
one GPU, equals one unsharded step of the whole model.

For each rank r: its slice of every rank's gradient is packed (contribution k
is rank k's own gradient over [r S, (r + 1) S)), the contributions are
averaged, and AdamW updates the slice's fp32 state, writing the bf16 copy
straight into the rank's window of one full flat parameter buffer (the
ZeRO-1/2 arrangement, where every rank ends up with all parameters).  The
persistent tensors take the AllReduce mean and the same update on every rank.
Unpacking the full buffer then gives per-tensor parameters that must equal, per
tensor, the oracle's plain step: the mean of the N_d gradients, then AdamW on
the whole tensor.  Bars as everywhere: the reduced gradient bit-exact; fp32
state within 1e-6 relative + 1e-9 absolute and bf16 parameters within 1 ulp,
and then bit for bit (the update is the oracle's double arithmetic).
"""
import numpy as np
import pytest
import torch

import oracle
import zero_sharded_optimizer_zr_amd as zr
from gpu_util import assert_bf16_exact, assert_bits_equal, assert_fp32_exact, device, say
from zr_workloads import TINY_MLP, synth

pytestmark = pytest.mark.gpu

HP = TINY_MLP.hparams
STEP = 3


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16).copy()


@pytest.mark.parametrize("numels,n_d,threshold", [
    (TINY_MLP.numels, 4, TINY_MLP.threshold),                     # the tiny MLP over 4 ranks, two persistent biases
    (TINY_MLP.numels, 3, TINY_MLP.threshold),                     # 3 ranks: tensors straddle shard edges, padding
    ([70_001, 13, 99_999, 100_000, 5_003, 131_071], 5, 100_000),  # threshold edges, ragged sizes
])
def test_all_ranks_equal_the_unsharded_step(numels, n_d, threshold):
    dev = device()
    say("all ranks", n_d, "ranks,", len(numels), "tensors")
    ref = oracle.Layout(numels, n_d, threshold)
    lay = zr.zr_layout_create(numels, n_d, threshold)
    S = ref.shard
    T = len(numels)
    # every rank's own per-tensor gradient, and the model's fp32 state before the step
    grads = [[synth.normal_bf16(x, 1e-3, synth.seed_of(50, t, 0, k), dev) for t, x in enumerate(numels)]
             for k in range(n_d)]
    theta = [synth.normal_f32(x, 0.02, synth.seed_of(51, t), dev) for t, x in enumerate(numels)]
    m0 = [synth.normal_f32(x, 1e-4, synth.seed_of(52, t), dev) for t, x in enumerate(numels)]
    v0 = [synth.uniform_f32(x, 1e-6, synth.seed_of(53, t), dev) for t, x in enumerate(numels)]
    before = [[a.cpu().numpy().copy() for a in (theta[t], m0[t], v0[t])] for t in range(T)]

    def flat_f32(per_tensor):
        """The partitioned tensors' fp32 values in list order, zero padded to Psi_pad."""
        parts = [per_tensor[t] for t in range(T) if not ref.persistent[t]]
        out = torch.zeros(ref.psi_pad, dtype=torch.float32, device=dev)
        if parts:
            cat = torch.cat(parts)
            out[:cat.numel()] = cat
        return out

    st = [flat_f32(x) for x in (theta, m0, v0)]
    full_param = torch.full((ref.psi_pad,), 0x7fc1, dtype=torch.int16, device=dev)
    full_grad = torch.empty(ref.psi_pad, dtype=torch.bfloat16, device=dev)
    for r in range(n_d):
        b, e = r * S, (r + 1) * S
        contribs = []
        for k in range(n_d):
            c = torch.empty(S, dtype=torch.bfloat16, device=dev)
            zr.zr_pack(lay, [None if ref.persistent[t] else grads[k][t] for t in range(T)], c, b, e)
            contribs.append(c)
        g = full_grad[b:e]
        zr.zr_reduce_slice(contribs, g)
        zr.zr_adamw_step(g, st[0][b:e], st[1][b:e], st[2][b:e], full_param[b:e], step=STEP, **HP)
    params = [torch.empty(x, dtype=torch.int16, device=dev) for x in numels]
    zr.zr_unpack(lay, full_param, 0, ref.psi_pad, [None if ref.persistent[t] else params[t] for t in range(T)])
    # persistent tensors: the AllReduce mean and the same update on every rank
    pers = [t for t in range(T) if ref.persistent[t]]
    for t in pers:
        g = torch.empty(numels[t], dtype=torch.bfloat16, device=dev)
        zr.zr_reduce_slice([grads[k][t] for k in range(n_d)], g)
        zr.zr_adamw_step(g, theta[t], m0[t], v0[t], params[t], step=STEP, **HP)
    torch.cuda.synchronize()

    # the oracle's unsharded step, tensor by tensor
    off = 0
    for t, x in enumerate(numels):
        mean = oracle.reduce([_bits(grads[k][t]) for k in range(n_d)])
        if ref.persistent[t]:
            got = [theta[t], m0[t], v0[t]]
        else:
            assert_bits_equal(_bits(full_grad[off:off + x]), mean, f"tensor {t} reduced gradient")
            got = [s[off:off + x] for s in st]
            off += x
        init = [a.copy() for a in before[t]]
        p = np.zeros(x, np.uint16)
        oracle.adamw(mean, *init, p, step=STEP, **HP)
        for name, a, want in zip(("master", "m", "v"), got, init):
            assert_fp32_exact(a.cpu().numpy(), want, f"tensor {t} {name}")
        assert_bf16_exact(params[t].cpu().numpy().view(np.uint16), p, f"tensor {t} param")
    # the padding of the last rank(s) stays zero state, and its parameter slots hold bf16 zeros
    pad = slice(ref.psi_part, ref.psi_pad)
    for s in st:
        assert not s[pad].any()
    assert_bits_equal(full_param[pad].cpu().numpy().view(np.uint16),
                      np.zeros(ref.psi_pad - ref.psi_part, np.uint16), "padding")
