"""Every element of the four full-size shards against the oracle.

The full-size shards of the 7e9 model over 4 ranks (the blog's "where 28 GB
comes from"), the Llama-style 7B and the GPT-style 7.5B over 64 ranks (the
hotelren.com article's 7.5B on 64 GPUs) and the 1T model over 512 ranks (the
encyclopedia entry's Applications) run the hot path's mean and AdamW calls on
the GPU, in the launch configuration the bench times.  Every output element --
the bf16 mean, fp32 master / m / v and the bf16 parameter copy -- is then
copied to the host chunk by chunk and compared with the oracle run over the
same chunk from the same inputs (the state as it was before the step), on all
host cores.  Bars: mean bit-exact; fp32 state within 1e-6 relative + 1e-9
absolute and bf16 copy within 1 ulp, then both bit for bit.  The GPT run checks each of its 10 steps
from the GPU's own state before that step.  The Llama shard's unpack into
per-tensor windows and the whole 13.5 GB flat-buffer pack are compared with
the oracle's unpack and pack over every element too.
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
import zero_sharded_optimizer_zr_amd as zr
from gpu_util import assert_bf16_exact, assert_bits_equal, assert_fp32_exact, device, say
from zr_workloads import FLAT_1T, FLAT_7B, GPT_7P5B, LLAMA_7B, synth

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

CHUNK_BYTES = 1 << 30   # host bytes of contributions per chunk
SUB = 1 << 20           # elements per host task


def _threads():
    return max(1, min(16, len(os.sched_getaffinity(0))))


@pytest.fixture(scope="module")
def pool():
    with ThreadPoolExecutor(_threads()) as p:
        yield p


@pytest.fixture(autouse=True)
def _free():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


class Pinned:
    """Pinned host staging for chunks of device tensors (fast, synchronous
    device -> host copies); one buffer per role, reused chunk after chunk."""

    def __init__(self):
        self.buf = {}

    def get(self, role, src: torch.Tensor) -> np.ndarray:
        n = src.numel()
        b = self.buf.get(role)
        if b is None or b.numel() < n or b.dtype != src.dtype:
            b = torch.empty(n, dtype=src.dtype, pin_memory=True)
            self.buf[role] = b
        h = b[:n]
        h.copy_(src)
        a = h.numpy()
        if a.dtype in (np.int16,):
            return a.view(np.uint16)
        return a


def u16v(t: torch.Tensor) -> torch.Tensor:
    return t.view(torch.int16)


def compare_step(pool, w, contribs, before, grad, state, param, step, what):
    """The oracle's mean and AdamW over every element, chunk by chunk, against
    the GPU's outputs; `before` holds device copies of master / m / v from
    before the step, `state` the updated ones."""
    n = grad.numel()
    nc = len(contribs)
    chunk = max(SUB, min(1 << 25, CHUNK_BYTES // (2 * nc)) // SUB * SUB)
    pin = Pinned()
    names = ("master", "exp_avg", "exp_avg_sq")
    for a in range(0, n, chunk):
        b = min(n, a + chunk)
        hc = [pin.get(f"c{k}", u16v(c)[a:b]) for k, c in enumerate(contribs)]
        hb = [pin.get(f"b{k}", before[k][a:b]) for k in range(3)]
        got_grad = pin.get("grad", u16v(grad)[a:b])
        got = [pin.get(f"s{k}", state[k][a:b]) for k in range(3)]
        got_param = pin.get("param", u16v(param)[a:b]) if param is not None else None
        o_grad = np.empty(b - a, np.uint16)
        o_param = np.empty(b - a, np.uint16) if param is not None else None

        def work(lo):
            hi = min(b - a, lo + SUB)
            sl = slice(lo, hi)
            oracle.reduce([x[sl] for x in hc], o_grad[sl])
            assert_bits_equal(got_grad[sl], o_grad[sl], f"{what} mean [{a + lo}, {a + hi})")
            # the oracle updates its own copies of the inputs in place
            st = [x[sl].copy() for x in hb]
            oracle.adamw(o_grad[sl], *st, None if o_param is None else o_param[sl], step=step, **w.hparams)
            for name, g, r in zip(names, got, st):
                assert_fp32_exact(g[sl], r, f"{what} {name} [{a + lo}, {a + hi})")
            if o_param is not None:
                assert_bf16_exact(got_param[sl], o_param[sl], f"{what} param [{a + lo}, {a + hi})")
            return hi - lo

        done = sum(pool.map(work, range(0, b - a, SUB)))
        assert done == b - a
    say(what, f"all {n} elements match the oracle")


def full_step(pool, w, n, steps, salt=0, param_out=True):
    """Shard state and contributions of workload w, the GPU mean and AdamW for
    each step of `steps`, every element compared after every step."""
    dev = device()
    st = synth.shard_state(w, n, device=dev, salt=salt)
    state = [st["master"], st["exp_avg"], st["exp_avg_sq"]]
    grad = torch.empty(n, dtype=torch.bfloat16, device=dev)
    param = torch.empty(n, dtype=torch.bfloat16, device=dev) if param_out else None
    for si, t in enumerate(steps):
        contribs = synth.contributions(w, n, step_index=si, device=dev, salt=salt)
        before = [x.clone() for x in state]
        say(w.name, f"step t={t}: {len(contribs)} contributions of {n}, mean + AdamW on the GPU")
        zr.zr_reduce_slice(contribs, grad)
        zr.zr_adamw_step(grad, *state, param, step=t, **w.hparams)
        torch.cuda.synchronize()
        compare_step(pool, w, contribs, before, grad, state, param, t, f"{w.name} t={t}")
        del contribs, before
        torch.cuda.empty_cache()
    return dict(state=state, grad=grad, param=param)


def test_full_flat_7b_nd4(pool):
    w = FLAT_7B
    lay = zr.zr_layout_create(w.numels, w.n_d, w.threshold)
    b, e = zr.zr_layout_rank_range(lay, w.rank)
    full_step(pool, w, e - b, w.steps)


def test_full_llama_7b_nd64_rank17(pool):
    w = LLAMA_7B
    dev = device()
    ref = oracle.Layout(w.numels, w.n_d, w.threshold)
    lay = zr.zr_layout_create(w.numels, w.n_d, w.threshold)
    b, e = zr.zr_layout_rank_range(lay, w.rank)
    out = full_step(pool, w, e - b, w.steps)
    # the updated shard unpacked into per-tensor windows: every element
    frs = ref.fragments(b, e)
    views = [None] * len(w.numels)
    for t, toff, _, n in frs:
        views[t] = (torch.full((n,), 0x5A5A, dtype=torch.int16, device=dev), toff)
    zr.zr_unpack(lay, out["param"], b, e, views)
    flat_h = out["param"].view(torch.int16).cpu().numpy().view(np.uint16)
    want = [None] * len(w.numels)
    for t, toff, _, n in frs:
        want[t] = (np.zeros(n, np.uint16), toff)
    oracle.unpack(ref, flat_h, b, e, want)
    for t, toff, _, n in frs:
        assert_bits_equal(views[t][0].cpu().numpy().view(np.uint16), want[t][0], f"llama r17 unpack tensor {t}")
    del out, views
    torch.cuda.empty_cache()
    # the persistent RMSNorm vectors: same update with no bf16 copy
    full_step(pool, w, ref.psi_persist, w.steps, salt=77, param_out=False)
    # the whole flat buffer packed from per-tensor views of random bits, every element
    say("llama: full-buffer pack of", ref.psi_pad, "elements, every element against the oracle")
    full_views = [None if ref.persistent[t] else synth.random_bits16(x, 500 + t, dev) for t, x in enumerate(w.numels)]
    flat = torch.empty(ref.psi_pad, dtype=torch.int16, device=dev)
    zr.zr_pack(lay, full_views, flat, 0, ref.psi_pad)
    for t in range(len(w.numels)):
        if ref.persistent[t]:
            continue
        off, n = ref.offset[t], w.numels[t]
        hv = full_views[t].cpu().numpy().view(np.uint16)
        hv_views = [None] * len(w.numels)
        hv_views[t] = (hv, 0)
        assert_bits_equal(flat[off:off + n].cpu().numpy().view(np.uint16), oracle.pack(ref, hv_views, off, off + n),
                          f"llama full pack tensor {t}")
    assert ref.psi_pad == ref.psi_part  # 64 divides it: no padding to check


def test_full_gpt_7p5b_nd64_ten_steps(pool):
    w = GPT_7P5B
    ref = oracle.Layout(w.numels, w.n_d, w.threshold)
    lay = zr.zr_layout_create(w.numels, w.n_d, w.threshold)
    b, e = zr.zr_layout_rank_range(lay, w.rank)
    full_step(pool, w, e - b, w.steps)
    full_step(pool, w, ref.psi_persist, w.steps, salt=55)


def test_full_flat_1t_nd512(pool):
    w = FLAT_1T
    lay = zr.zr_layout_create(w.numels, w.n_d, w.threshold)
    b, e = zr.zr_layout_rank_range(lay, w.rank)
    out = full_step(pool, w, e - b, w.steps)
    # the full unpack of the shard into the tensor's window [b, e): the oracle's
    # unpack of a one-tensor layout is the identity, so every element must equal
    # the flat shard
    view = torch.empty(e - b, dtype=torch.bfloat16, device=device())
    zr.zr_unpack(lay, out["param"], b, e, [(view, b)])
    assert torch.equal(view.view(torch.int16), out["param"].view(torch.int16))


# ---------------------------------------------------------------- NEXT paths --

def _chunks(n, size):
    return [(a, min(n, a + size)) for a in range(0, n, size)]


def test_full_fp16_flat_7b_nd4(pool):
    """The fp16 path with dynamic loss scaling on the 7e9 / N_d = 4 shard (the
    tutorial's fp16 config, cnhsyj.com 3.1: scale 2^16): the fp16 mean of 4
    loss-scaled contributions and the loss-scaled AdamW with its fp16 copy, every
    element against the oracle's reduce_f16 and adamw_f16 (mean bit-exact, state
    and copy bit-exact after the bars)."""
    dev = device()
    w = FLAT_7B
    lay = zr.zr_layout_create(w.numels, w.n_d, w.threshold)
    b0, e0 = zr.zr_layout_rank_range(lay, w.rank)
    n = e0 - b0
    scale = 65536.0
    contribs = [synth.normal_f32(n, 1e-3 * scale, 900 + k, dev).to(torch.float16) for k in range(4)]
    st = synth.shard_state(w, n, device=dev)
    state = [st["master"], st["exp_avg"], st["exp_avg_sq"]]
    before = [x.clone() for x in state]
    ls = zr.loss_scale_record(dev)
    zr.zr_loss_scale_init(ls, scale)
    grad = torch.empty(n, dtype=torch.float16, device=dev)
    param = torch.empty(n, dtype=torch.float16, device=dev)
    say("fp16: mean of 4 contributions and loss-scaled AdamW on", n, "elements")
    zr.zr_reduce_slice_f16(contribs, grad, ls)
    zr.zr_adamw_step_f16(grad, *state, param, ls, step=w.steps[0], **w.hparams)
    torch.cuda.synchronize()
    assert int(ls.cpu()[2]) == 0, "no overflow expected"
    pin = Pinned()
    names = ("master", "exp_avg", "exp_avg_sq")
    for a, b in _chunks(n, 1 << 25):
        hc = [pin.get(f"c{k}", u16v(c)[a:b]) for k, c in enumerate(contribs)]
        hb = [pin.get(f"b{k}", before[k][a:b]) for k in range(3)]
        got_grad = pin.get("grad", u16v(grad)[a:b])
        got = [pin.get(f"s{k}", state[k][a:b]) for k in range(3)]
        got_param = pin.get("param", u16v(param)[a:b])

        def work(lo, a=a, b=b, hc=hc, hb=hb, got_grad=got_grad, got=got, got_param=got_param):
            hi = min(b - a, lo + SUB)
            sl = slice(lo, hi)
            o_grad = oracle.reduce_f16([x[sl] for x in hc])
            assert_bits_equal(got_grad[sl], o_grad, f"fp16 mean [{a + lo}, {a + hi})")
            st_ = [x[sl].copy() for x in hb]
            o_param = np.empty(hi - lo, np.uint16)
            oracle.adamw_f16(o_grad, *st_, o_param, step=w.steps[0], loss_scale=scale, **w.hparams)
            for name, g, r in zip(names, got, st_):
                assert_fp32_exact(g[sl], r, f"fp16 {name} [{a + lo}, {a + hi})")
            assert_bits_equal(got_param[sl], o_param, f"fp16 copy [{a + lo}, {a + hi})")
            return hi - lo

        assert sum(pool.map(work, range(0, b - a, SUB))) == b - a
    say("fp16: all", n, "elements match the oracle")


def _random_codes(nbytes, int4, seed, dev):
    """Codes of the other ranks' shards: int8 in [-127, 127], or int4 nibble
    pairs in [-7, 7] (never the pattern 8)."""
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    if int4:
        lo = torch.randint(-7, 8, (nbytes,), generator=g, device=dev, dtype=torch.int16) & 0xF
        hi = torch.randint(-7, 8, (nbytes,), generator=g, device=dev, dtype=torch.int16) & 0xF
        return (lo | (hi << 4)).to(torch.uint8)
    return torch.randint(-127, 128, (nbytes,), generator=g, device=dev, dtype=torch.int8)


@pytest.mark.parametrize("int4", [False, True], ids=["int8", "int4"])
def test_full_qwz_gather_flat_7b_nd4(pool, int4):
    """The quantized AllGather (ZeRO++ qwZ on the concept page,
    compassingai.com) on the 7e9 model over 4 ranks, block 2048: rank 0
    quantizes its whole 1.75e9-element bf16 shard in one call (codes and block
    scales of every block, the short last block included, against the oracle's
    quantize over each block-aligned chunk), and the gathered 7e9 elements (rank
    0's codes and three ranks of random codes) are rebuilt into the tensor's
    bf16 view in one call, every element against the oracle's gathered unpack."""
    dev = device()
    B = 2048
    w = FLAT_7B
    lay = zr.zr_layout_create(w.numels, w.n_d, w.threshold)
    ref = oracle.Layout(w.numels, w.n_d, w.threshold)
    S, G = ref.shard, ref.psi_pad
    per_rank = -(-S // B)
    bytes_per_rank = -(-S // 2) if int4 else S
    x = synth.normal_bf16(S, 0.02, 4242, dev)
    codes = torch.empty(w.n_d * bytes_per_rank, dtype=torch.uint8 if int4 else torch.int8, device=dev)
    scales = torch.empty(w.n_d * per_rank, dtype=torch.float32, device=dev)
    quant = zr.zr_quantize_int4 if int4 else zr.zr_quantize_int8
    say("qwz", "int4" if int4 else "int8", ": quantize the", S, "element shard")
    quant(x, codes[:bytes_per_rank], scales[:per_rank], block=B)
    torch.cuda.synchronize()
    # rank 0's codes and scales: every block against the oracle
    pin = Pinned()
    oq = oracle.quantize_int4 if int4 else oracle.quantize_int8
    chunk = (1 << 24) // B * B
    hx = x.view(torch.int16)
    for a, b in _chunks(S, chunk):
        xs = pin.get("x", hx[a:b])
        ca, cb = (a // 2, -(-b // 2)) if int4 else (a, b)
        got_q = pin.get("q", codes[ca:cb])
        got_s = pin.get("s", scales[a // B: -(-b // B)])

        def work(lo, a=a, b=b, xs=xs, got_q=got_q, got_s=got_s):
            hi = min(b - a, lo + SUB)     # SUB is a multiple of B and even
            q, s = oq(np.ascontiguousarray(xs[lo:hi]), B)
            qs = slice(lo // 2, lo // 2 + q.size) if int4 else slice(lo, hi)
            assert_bits_equal(np.ascontiguousarray(got_q[qs]).view(np.uint8), q.view(np.uint8),
                              f"codes [{a + lo}, {a + hi})")
            assert_bits_equal(np.ascontiguousarray(got_s[lo // B: lo // B + s.size]), s,
                              f"scales [{a + lo}, {a + hi})")
            return hi - lo

        assert sum(pool.map(work, range(0, b - a, SUB))) == b - a
    # the gathered buffer: ranks 1..3 random codes and positive scales
    codes[bytes_per_rank:] = _random_codes(3 * bytes_per_rank, int4, 77, dev).view(codes.dtype)
    scales[per_rank:] = synth.uniform_f32(3 * per_rank, 1e-3, 78, dev) + 1e-4
    view = torch.empty(G, dtype=torch.bfloat16, device=dev)
    unpack = zr.zr_unpack_int4 if int4 else zr.zr_unpack_int8
    say("qwz: rebuild the", G, "gathered elements into the view")
    unpack(lay, codes, scales, 0, G, [view], block=B)
    torch.cuda.synchronize()
    ou = oracle.unpack_int4 if int4 else oracle.unpack_int8
    hv = view.view(torch.int16)
    for r in range(w.n_d):
        for a, b in _chunks(S, chunk):
            fa, fb = r * S + a, r * S + b
            ca, cb = ((r * bytes_per_rank + a // 2, r * bytes_per_rank + -(-b // 2)) if int4
                      else (fa, fb))
            got = pin.get("v", hv[fa:fb])
            hq = pin.get("q", codes[ca:cb])
            hs = pin.get("s", scales[r * per_rank + a // B: r * per_rank + -(-b // B)])

            def work(lo, fa=fa, fb=fb, got=got, hq=hq, hs=hs):
                hi = min(fb - fa, lo + SUB)
                out = np.zeros(hi - lo, np.uint16)
                qs = slice(lo // 2, -(-hi // 2)) if int4 else slice(lo, hi)
                q = np.ascontiguousarray(hq[qs]).view(np.uint8 if int4 else np.int8)
                ou(ref, q, np.ascontiguousarray(hs[lo // B: -(-hi // B)]), B, fa + lo, fa + hi, [(out, fa + lo)])
                assert_bits_equal(got[lo:hi], out, f"rebuilt [{fa + lo}, {fa + hi})")
                return hi - lo

            assert sum(pool.map(work, range(0, fb - fa, SUB))) == fb - fa
    say("qwz: all", G, "rebuilt elements match the oracle")
