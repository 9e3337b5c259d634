"""Several host threads drive the library at once, each on its own stream and
buffers (one layout object shared by all): every thread's step results equal
the same steps run alone, bit for bit, and each thread's zr_last_error() holds
only its own failures."""
import threading

import numpy as np
import pytest
import torch

import zero_sharded_optimizer_zr_amd as zr
from gpu_util import device, say
from zr_workloads import TINY_MLP, synth

pytestmark = pytest.mark.gpu

THREADS = 4
STEPS = 5


def _setup(dev, lay, seed):
    w = TINY_MLP
    b, e = zr.zr_layout_rank_range(lay, 1)
    S = e - b
    frags = zr.zr_layout_fragments(lay, b, e)
    own = [None] * len(w.numels)
    params = [None] * len(w.numels)
    for t, toff, _, cnt in frags:
        own[t] = (synth.normal_bf16(cnt, 1e-3, seed + t, dev), toff)
        params[t] = (torch.zeros(cnt, dtype=torch.int16, device=dev), toff)
    contribs = [torch.empty(S, dtype=torch.bfloat16, device=dev)] + \
        [synth.normal_bf16(S, 1e-3, seed + 100 + k, dev) for k in range(1, 4)]
    st = synth.shard_state(w, S, device=dev, salt=seed)
    return dict(b=b, e=e, own=own, params=params, contribs=contribs, grad=torch.empty(S, dtype=torch.bfloat16, device=dev),
                state=[st[k].clone() for k in ("master", "exp_avg", "exp_avg_sq")],
                flat=torch.zeros(S, dtype=torch.int16, device=dev))


def _steps(lay, s, stream):
    for t in range(1, STEPS + 1):
        zr.zr_pack(lay, s["own"], s["contribs"][0], s["b"], s["e"], stream=stream)
        zr.zr_reduce_slice(s["contribs"], s["grad"], stream=stream)
        zr.zr_adamw_step(s["grad"], *s["state"], s["flat"], step=t, stream=stream, **TINY_MLP.hparams)
        zr.zr_unpack(lay, s["flat"], s["b"], s["e"], s["params"], stream=stream)


def _result(s):
    return [x.cpu().numpy().view(np.uint32 if x.dtype == torch.float32 else np.uint16).copy()
            for x in s["state"] + [s["flat"]] + [p[0] for p in s["params"] if p is not None]]


def test_threads_on_their_own_streams_match_the_serial_run():
    dev = device()
    w = TINY_MLP
    lay = zr.zr_layout_create(w.numels, w.n_d, w.threshold)
    seeds = [1000 * (k + 1) for k in range(THREADS)]
    # serial reference
    want = []
    for sd in seeds:
        s = _setup(dev, lay, sd)
        _steps(lay, s, torch.cuda.current_stream())
        torch.cuda.synchronize()
        want.append(_result(s))
    # the same work from THREADS threads at once
    states = [_setup(dev, lay, sd) for sd in seeds]
    streams = [torch.cuda.Stream() for _ in seeds]
    torch.cuda.synchronize()
    errors, messages = [], {}
    barrier = threading.Barrier(THREADS)

    def worker(k):
        try:
            torch.cuda.set_device(dev)
            barrier.wait()
            with torch.cuda.stream(streams[k]):
                _steps(lay, states[k], streams[k])
                # a failure on this thread only: its message must name this call
                try:
                    zr.zr_reduce_slice([], states[k]["grad"], stream=streams[k])
                except zr.ZRError as e:
                    messages[k] = (e.status, zr.zr_last_error())
        except Exception as e:  # noqa: BLE001 -- reported below
            errors.append(repr(e))

    threads = [threading.Thread(target=worker, args=(k,)) for k in range(THREADS)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=120)
    assert not any(th.is_alive() for th in threads), "a worker thread did not finish"
    torch.cuda.synchronize()
    assert not errors, errors
    for k in range(THREADS):
        say("thread", k)
        for a, b in zip(_result(states[k]), want[k]):
            assert np.array_equal(a, b), f"thread {k} differs from the serial run"
        status, msg = messages[k]
        assert status == zr.ZR_EINVAL and "zr_reduce_slice" in msg, (status, msg)
    # the main thread saw none of the workers' failures
    assert zr.zr_last_error() == ""
