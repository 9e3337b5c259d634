"""GPU tests of the ZeRO-Offload step (zr_offload_adamw_step): device bf16
gradient -> host AdamW on host fp32 states -> device bf16 parameters, through a
pinned staging buffer in chunks.  The results must equal the GPU AdamW kernel
(zr_adamw_step) bit for bit -- the host performs the same double operations
in the same order -- and the oracle bit for bit; chunk edges, ragged tails, a missing
parameter copy, stream order after the kernel that produced the gradient, and
the full 1.75e9-element shard."""
import numpy as np
import pytest
import torch

import oracle
import zero_sharded_optimizer_zr_amd as zr
from gpu_util import assert_bf16_exact, assert_fp32_exact, device, say
from zr_workloads import FLAT_7B, synth

pytestmark = pytest.mark.gpu

HP = dict(lr=5e-5, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)


def host_state(n, seed):
    rng = np.random.default_rng(seed)
    return (rng.normal(0, 0.02, n).astype(np.float32), rng.normal(0, 1e-4, n).astype(np.float32),
            rng.uniform(0, 1e-6, n).astype(np.float32))


def bits(t):
    return t.cpu().numpy().view(np.uint32 if t.dtype == torch.float32 else np.uint16)


def run_both(n, staging_bytes, step=10, with_param=True, seed=0, **kw):
    dev = device()
    rng = np.random.default_rng(seed)
    g = oracle.bf16_from_f32(rng.normal(0, 1e-3, n).astype(np.float32))
    th, m, v = host_state(n, seed + 1)
    grad = torch.from_numpy(g.view(np.int16)).to(dev)
    # GPU reference step
    gs = [torch.from_numpy(x.copy()).to(dev) for x in (th, m, v)]
    gp = torch.zeros(n, dtype=torch.int16, device=dev)
    zr.zr_adamw_step(grad, *gs, gp, step=step, **{**HP, **kw})
    # offloaded step
    hs = [torch.from_numpy(x.copy()) for x in (th, m, v)]
    op = torch.full((n,), 0x1234, dtype=torch.int16, device=dev) if with_param else None
    staging = zr.offload_staging(staging_bytes)
    zr.zr_offload_adamw_step(grad, *hs, op, staging, step=step, **{**HP, **kw})
    torch.cuda.synchronize()
    return (g, th, m, v), gs, gp, hs, op


@pytest.mark.parametrize("n,staging", [(1, 65536), (8191, 65536), (8192, 65536), (8193, 65536),
                                       (100_003, 65536), (1_000_003, 1 << 20), (3_000_000, 64 << 20)])
def test_offload_equals_gpu_adamw_bit_for_bit(n, staging):
    say("offload n", n, "staging", staging)
    _, gs, gp, hs, op = run_both(n, staging, seed=n)
    for name, a, b in zip(("master", "m", "v"), hs, gs):
        assert np.array_equal(bits(a), bits(b)), name
    assert np.array_equal(bits(op), bits(gp)), "param"


@pytest.mark.parametrize("step,kw", [(1, {}), (1000, dict(lr=1e-4, weight_decay=0.1)), (5, dict(grad_scale=0.125))])
def test_offload_matches_oracle(step, kw):
    n = 200_003
    (g, th, m, v), _, _, hs, op = run_both(n, 65536 * 4, step=step, seed=step, **kw)
    ref = [th.copy(), m.copy(), v.copy()]
    rp = np.zeros(n, np.uint16)
    oracle.adamw(g, *ref, rp, step=step, **{**HP, **kw})
    for name, a, b in zip(("master", "m", "v"), hs, ref):
        assert_fp32_exact(a.numpy(), b, f"offload {name}")
    assert_bf16_exact(bits(op), rp, "offload param")


def test_offload_without_param_copy():
    n = 50_000
    _, gs, _, hs, _ = run_both(n, 65536, with_param=False, seed=3)
    for a, b in zip(hs, gs):
        assert np.array_equal(bits(a), bits(b))


def test_offload_follows_the_stream_order_of_the_gradient():
    """The reduce that produces the gradient is still queued on the stream when
    the offloaded step starts: the step must see the reduced gradient."""
    dev = device()
    n = 2_000_003
    contribs = [synth.normal_bf16(n, 1e-3, 500 + k, dev) for k in range(8)]
    grad = torch.empty(n, dtype=torch.bfloat16, device=dev)
    th, m, v = host_state(n, 11)
    torch.cuda.synchronize()
    zr.zr_reduce_slice(contribs, grad)               # enqueued, not waited for
    hs = [torch.from_numpy(x.copy()) for x in (th, m, v)]
    op = torch.empty(n, dtype=torch.int16, device=dev)
    zr.zr_offload_adamw_step(grad, *hs, op, zr.offload_staging(1 << 20), step=2, **HP)
    gs = [torch.from_numpy(x.copy()).to(dev) for x in (th, m, v)]
    gp = torch.empty(n, dtype=torch.int16, device=dev)
    zr.zr_adamw_step(grad, *gs, gp, step=2, **HP)
    torch.cuda.synchronize()
    for a, b in zip(hs, gs):
        assert np.array_equal(bits(a), bits(b))
    assert np.array_equal(bits(op), bits(gp))


def test_offload_refuses_a_capturing_stream():
    """The offloaded step waits for its own copies, so a call on a stream that
    is being captured is rejected before anything is enqueued."""
    dev = device()
    n = 4096
    grad = torch.zeros(n, dtype=torch.int16, device=dev)
    hs = [torch.zeros(n, dtype=torch.float32) for _ in range(3)]
    staging = zr.offload_staging(1 << 20)
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        zr.zr_graph_capture_begin()
        with pytest.raises(zr.ZRError) as e:
            zr.zr_offload_adamw_step(grad, *hs, None, staging, step=1, **HP)
        zr.zr_reduce_slice([grad.view(torch.bfloat16)], grad.view(torch.bfloat16))   # something to capture
        g = zr.zr_graph_capture_end()
    zr.zr_graph_destroy(g)
    assert e.value.status == zr.ZR_EINVAL and "captured" in str(e.value)
    assert all(not h.any() for h in hs)


@pytest.mark.slow
def test_offload_full_shard_7b_over_4_ranks():
    """The 1.75e9-element shard of a 7e9-parameter model over 4 ranks: host
    states of 21 GB, one offloaded step against the GPU kernel, bit for bit."""
    dev = device()
    w = FLAT_7B
    S = w.numels[0] // w.n_d
    say("offload full shard", S)
    st = synth.shard_state(w, S, device=dev)
    grad = synth.normal_bf16(S, w.grad_std, synth.seed_of(w.seed, 60), dev)
    hs = [st[k].cpu() for k in ("master", "exp_avg", "exp_avg_sq")]
    op = torch.empty(S, dtype=torch.int16, device=dev)
    gp = torch.empty(S, dtype=torch.int16, device=dev)
    zr.zr_offload_adamw_step(grad, *hs, op, zr.offload_staging(64 << 20), step=w.steps[0], **w.hparams)
    zr.zr_adamw_step(grad, st["master"], st["exp_avg"], st["exp_avg_sq"], gp, step=w.steps[0], **w.hparams)
    torch.cuda.synchronize()
    for name, a in zip(("master", "exp_avg", "exp_avg_sq"), hs):
        assert torch.equal(a.view(torch.int32), st[name].cpu().view(torch.int32)), name
    assert torch.equal(op, gp)
    del st, grad, hs, op, gp
    torch.cuda.empty_cache()
