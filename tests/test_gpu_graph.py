"""GPU tests of captured steps (zr_graph_*): the four-call step, the fused
path and the fp16 path recorded once and replayed with new AdamW
hyper-parameters each step must give, after every replay, the same bits as the
same calls made eagerly on a copy of the state.  Every test replays several
times with eager torch work and synchronisation between the replays.  The
GPT-7.5B shard (N_d = 64, rank 0) runs its 10 steps with fresh gradient
contributions copied into the recorded buffers before each replay."""
import numpy as np
import pytest
import torch

import zero_sharded_optimizer_zr_amd as zr
from gpu_util import device, say
from zr_workloads import GPT_7P5B, TINY_MLP, synth

pytestmark = pytest.mark.gpu


def eq(a, b):
    return torch.equal(a.view(torch.int32) if a.dtype == torch.float32 else a.view(torch.int16),
                       b.view(torch.int32) if b.dtype == torch.float32 else b.view(torch.int16))


class Shard:
    """One rank's step buffers for workload w: own-gradient views, contributions
    (contribs[0] is the packed own gradient), the reduced gradient, the state,
    the flat parameter slot and the parameter views."""

    def __init__(self, w, dev, seed, state=None):
        self.lay = zr.zr_layout_create(w.numels, w.n_d, w.threshold)
        self.b, self.e = zr.zr_layout_rank_range(self.lay, w.rank)
        S = self.e - self.b
        self.frags = zr.zr_layout_fragments(self.lay, self.b, self.e)
        self.own = [None] * len(w.numels)
        self.params = [None] * len(w.numels)
        for t, toff, _, cnt in self.frags:
            self.own[t] = (synth.normal_bf16(cnt, w.grad_std, seed + t, dev), toff)
            self.params[t] = (torch.zeros(cnt, dtype=torch.int16, device=dev), toff)
        self.contribs = [torch.empty(S, dtype=torch.bfloat16, device=dev)] + \
            [synth.normal_bf16(S, w.grad_std, seed + 1000 + k, dev) for k in range(1, w.n_contrib)]
        self.grad = torch.empty(S, dtype=torch.bfloat16, device=dev)
        st = state if state is not None else synth.shard_state(w, S, device=dev)
        self.st = [st[k].clone() for k in ("master", "exp_avg", "exp_avg_sq")]
        self.flat = torch.zeros(S, dtype=torch.int16, device=dev)

    def copy_inputs_from(self, o):
        for (a, _), (b, _) in zip([x for x in self.own if x], [x for x in o.own if x]):
            a.copy_(b)
        for a, b in zip(self.contribs[1:], o.contribs[1:]):
            a.copy_(b)

    def step_calls(self, hp, step, stream):
        zr.zr_pack(self.lay, self.own, self.contribs[0], self.b, self.e, stream=stream)
        zr.zr_reduce_slice(self.contribs, self.grad, stream=stream)
        zr.zr_adamw_step(self.grad, *self.st, self.flat, step=step, stream=stream, **hp)
        zr.zr_unpack(self.lay, self.flat, self.b, self.e, self.params, stream=stream)

    def same_as(self, o):
        return (all(eq(a, b) for a, b in zip(self.st, o.st)) and eq(self.flat, o.flat) and
                all(eq(a[0], b[0]) for a, b in zip([x for x in self.params if x], [x for x in o.params if x])))


def test_captured_step_matches_eager_every_step():
    dev = device()
    w = TINY_MLP
    eager = Shard(w, dev, 11)
    rec = Shard(w, dev, 11, state={"master": eager.st[0], "exp_avg": eager.st[1], "exp_avg_sq": eager.st[2]})
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        zr.zr_graph_capture_begin()
        rec.step_calls(w.hparams, 1, None)
        g = zr.zr_graph_capture_end()
    kernels, adamw = zr.zr_graph_info(g)
    assert adamw == 1 and kernels >= 4
    # recording enqueued nothing
    torch.cuda.synchronize()
    assert not rec.flat.any()
    x = torch.ones(1 << 20, device=dev)
    for t in range(1, 7):
        say("captured step", t)
        eager.step_calls(w.hparams, t, torch.cuda.current_stream())
        zr.zr_graph_set_adamw(g, step=t, **w.hparams)
        zr.zr_graph_launch(g, side)
        x.mul_(1.0001)                                   # eager work between the replays
        torch.cuda.synchronize()
        assert rec.same_as(eager), f"step {t}"
    zr.zr_graph_destroy(g)


def test_captured_fused_and_fp16_paths_with_an_overflow():
    dev = device()
    w = TINY_MLP
    S = 262_144
    hp = w.hparams
    side = torch.cuda.Stream()
    # fused reduce + AdamW
    contribs = [synth.normal_bf16(S, 1e-3, 50 + k, dev) for k in range(4)]
    base = synth.shard_state(w, S, device=dev)
    a = [base[k].clone() for k in ("master", "exp_avg", "exp_avg_sq")]
    b = [base[k].clone() for k in ("master", "exp_avg", "exp_avg_sq")]
    pa, pb = torch.zeros(S, dtype=torch.int16, device=dev), torch.zeros(S, dtype=torch.int16, device=dev)
    # fp16 path
    scale = 2.0 ** 16
    c16 = [synth.normal_f32(S, 1e-3 * scale, 60 + k, dev).to(torch.float16) for k in range(4)]
    g16a, g16b = torch.empty(S, dtype=torch.float16, device=dev), torch.empty(S, dtype=torch.float16, device=dev)
    fa = [base[k].clone() for k in ("master", "exp_avg", "exp_avg_sq")]
    fb = [base[k].clone() for k in ("master", "exp_avg", "exp_avg_sq")]
    qa, qb = torch.zeros(S, dtype=torch.int16, device=dev), torch.zeros(S, dtype=torch.int16, device=dev)
    lsa, lsb = zr.loss_scale_record(dev), zr.loss_scale_record(dev)
    zr.zr_loss_scale_init(lsa, scale)
    zr.zr_loss_scale_init(lsb, scale)
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        zr.zr_graph_capture_begin()
        zr.zr_reduce_adamw_step(contribs, *b, pb, step=1, **hp)
        zr.zr_reduce_slice_f16(c16, g16b, lsb)
        zr.zr_adamw_step_f16(g16b, *fb, qb, lsb, step=1, **hp)
        zr.zr_loss_scale_update(lsb)
        g = zr.zr_graph_capture_end()
    assert zr.zr_graph_info(g)[1] == 2
    for t in range(1, 6):
        say("captured fused/fp16 step", t)
        if t == 3:
            c16[1][777] = float("inf")                   # an overflowing backward in step 3
        if t == 4:
            c16[1][777] = 1.0
        zr.zr_reduce_adamw_step(contribs, *a, pa, step=t, **hp)
        zr.zr_reduce_slice_f16(c16, g16a, lsa)
        zr.zr_adamw_step_f16(g16a, *fa, qa, lsa, step=t, **hp)
        zr.zr_loss_scale_update(lsa)
        zr.zr_graph_set_adamw(g, step=t, **hp)
        zr.zr_graph_launch(g, side)
        torch.cuda.synchronize()
        assert all(eq(x, y) for x, y in zip(a, b)) and eq(pa, pb), f"fused step {t}"
        assert all(eq(x, y) for x, y in zip(fa, fb)) and eq(qa, qb), f"fp16 step {t}"
        assert torch.equal(lsa, lsb), f"loss-scale record step {t}"
    assert int(lsb.cpu()[3]) == 1                        # the overflowing step was skipped
    zr.zr_graph_destroy(g)


@pytest.mark.parametrize("bits", [8, 4])
def test_captured_step_with_a_quantized_gather(bits):
    """A step that ends in the quantized AllGather's local halves -- AdamW, the
    rank's own shard quantized into its slot of the gathered codes, then the
    whole gathered range rebuilt into the views -- recorded once and replayed,
    equal to the eager calls after every replay."""
    dev = device()
    w = TINY_MLP
    block = 256
    lay = zr.zr_layout_create(w.numels, w.n_d, w.threshold)
    info = zr.zr_layout_query(lay)
    S, G = info["shard"], info["psi_pad"]
    per_rank = -(-S // block)
    nbytes = S if bits == 8 else -(-S // 2)
    quantize = zr.zr_quantize_int8 if bits == 8 else zr.zr_quantize_int4
    unpack = zr.zr_unpack_int8 if bits == 8 else zr.zr_unpack_int4
    ctype = torch.int8 if bits == 8 else torch.uint8

    def buffers(seed):
        g = synth.normal_bf16(S, 1e-3, seed, dev)
        st = [x.clone() for x in synth.shard_state(w, S, device=dev).values()]
        flat = torch.zeros(S, dtype=torch.int16, device=dev)
        gen = torch.Generator(device=dev)
        gen.manual_seed(seed)
        codes = torch.randint(-7, 8, (w.n_d * nbytes,), dtype=torch.int8, device=dev, generator=gen).view(ctype)
        scales = torch.rand(w.n_d * per_rank, dtype=torch.float32, device=dev, generator=gen) * 1e-3
        views = [None if zr.zr_layout_tensor(lay, t)[0] else torch.zeros(x, dtype=torch.int16, device=dev)
                 for t, x in enumerate(w.numels)]
        return g, st, flat, codes, scales, views

    def calls(bf, step, stream):
        g, st, flat, codes, scales, views = bf
        zr.zr_adamw_step(g, *st, flat, step=step, stream=stream, **w.hparams)
        quantize(flat, codes[:nbytes], scales[:per_rank], block=block, stream=stream)
        unpack(lay, codes, scales, 0, G, views, block=block, stream=stream)

    eager, rec = buffers(31), buffers(31)
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        zr.zr_graph_capture_begin()
        calls(rec, 1, None)
        g = zr.zr_graph_capture_end()
    assert zr.zr_graph_info(g)[1] == 1
    for t in range(1, 4):
        say("captured quantized-gather step", bits, t)
        calls(eager, t, torch.cuda.current_stream())
        zr.zr_graph_set_adamw(g, step=t, **w.hparams)
        zr.zr_graph_launch(g, side)
        torch.cuda.synchronize()
        for a, b in zip(eager[1] + [eager[2], eager[3].view(torch.int8), eager[4]],
                        rec[1] + [rec[2], rec[3].view(torch.int8), rec[4]]):
            assert eq(a, b) if a.dtype != torch.int8 else torch.equal(a, b), f"step {t}"
        for a, b in zip(eager[5], rec[5]):
            assert a is None or torch.equal(a, b), f"views, step {t}"
    zr.zr_graph_destroy(g)


@pytest.mark.slow
def test_captured_gpt_shard_ten_steps_with_fresh_contributions():
    """The GPT-7.5B shard over 64 ranks (116,465,664 elements, 435 tensors),
    10 consecutive steps, fresh contributions every step copied into the
    recorded buffers; the recorded step equals the eager one after every step."""
    dev = device()
    w = GPT_7P5B
    eager = Shard(w, dev, 21)
    rec = Shard(w, dev, 21, state={"master": eager.st[0], "exp_avg": eager.st[1], "exp_avg_sq": eager.st[2]})
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        zr.zr_graph_capture_begin()
        rec.step_calls(w.hparams, 1, None)
        g = zr.zr_graph_capture_end()
    S = eager.e - eager.b
    for t in w.steps:
        fresh = synth.contributions(w, S, step_index=t - 1, device=dev)
        for k in range(1, w.n_contrib):
            eager.contribs[k].copy_(fresh[k])
            rec.contribs[k].copy_(fresh[k])
        del fresh
        torch.cuda.synchronize()
        eager.step_calls(w.hparams, t, torch.cuda.current_stream())
        zr.zr_graph_set_adamw(g, step=t, **w.hparams)
        zr.zr_graph_launch(g, side)
        torch.cuda.synchronize()
        assert rec.same_as(eager), f"step {t}"
    zr.zr_graph_destroy(g)
