"""Calls on different streams from different host threads at once.

The library keeps no mutable global state and a call's only device state is its caller's
workspace, so calls on different streams with different workspaces may run together.  Four
host threads each repeat one call on a stream and workspace of their own: two 512-token
layers on different inputs (routing, then the paired GEMM launch whose workgroups wait on
each other's tiles, so two such launches share the chip), the decode-sized layer at 4
tokens (workgroups that wait on earlier ones' flags), and GQA decode attention over 32K
positions.  Each result must equal the same call made alone, bit
for bit, every time, and no bounded wait may have given up (the layers' error word).
"""
import threading

import numpy as np
import pytest

from bit_grouped_expert_amd import _lib as L
from bit_grouped_expert_amd import device as dev
from bit_grouped_expert_amd import workload as wl

pytestmark = pytest.mark.gpu

ROUNDS = 30


def say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    L.lib()
    return torch


def test_concurrent_streams_and_threads(torch_cuda):
    torch = torch_cuda
    cfg = wl.CONFIGS["prefill512"]
    lw = dev.LayerWeights(wl.make_weights(cfg, wl.layer_seed(0)), cfg.E)
    jobs = []

    def layer_job(T, seed):
        shp = L.shape(T, cfg.D, cfg.E, cfg.k, cfg.F)
        x, r = wl.make_activations(wl.MoEConfig(f"conc{T}", T, cfg.D, cfg.E, cfg.k, cfg.F), seed)
        xd, rd = dev.to_device(x), dev.to_device(r)
        ws = dev.workspace(shp)
        out = torch.empty((T, cfg.D), dtype=torch.int16, device="cuda")
        lay = L.moe_workspace_layout(shp)

        def run(stream):
            L.moe_layer_forward(shp, xd, rd, lw.experts, lw.shared, out, ws, stream=stream)

        def error_word():
            return int(ws[lay.sync:lay.sync + 4].cpu().numpy().view(np.int32)[0])
        return f"layer T={T} (inputs {seed})", run, out, error_word

    def attention_job(ctx):
        q, k, v = wl.make_attention_inputs(16, 2, 128, ctx, None, 3, 1.0)
        shp = L.gqa_shape(16, 2, 128, ctx, None)
        qd, kd, vd = dev.to_device(q), dev.to_device(k), dev.to_device(v)
        ws = torch.empty(L.moe_gqa_decode_workspace_bytes(shp), dtype=torch.uint8, device="cuda")
        out = torch.empty((16, 128), dtype=torch.int16, device="cuda")

        def run(stream):
            L.moe_gqa_decode_attention(shp, qd, kd, vd, out, ws, stream=stream)
        return f"attention ctx={ctx}", run, out, lambda: 0

    jobs = [layer_job(512, 0), layer_job(512, 2), layer_job(4, 1), attention_job(32768)]
    # each call alone first
    refs = []
    for name, run, out, err in jobs:
        run(torch.cuda.current_stream())
        torch.cuda.synchronize()
        assert err() == 0, f"{name}: a wait gave up when run alone"
        refs.append(out.clone())
    failures = []

    def worker(i):
        name, run, out, err = jobs[i]
        s = torch.cuda.Stream()
        try:
            for rnd in range(ROUNDS):
                with torch.cuda.stream(s):
                    out.fill_(0)
                    run(s)
                s.synchronize()
                if not torch.equal(out, refs[i]):
                    failures.append(f"{name}: round {rnd} differs from the call made alone")
                    return
                if err() != 0:
                    failures.append(f"{name}: round {rnd}: {err()} waits gave up")
                    return
        except Exception as e:  # noqa: BLE001 - reported below
            failures.append(f"{name}: {e!r}")

    say(f"{len(jobs)} host threads, {ROUNDS} rounds each, one stream and workspace per thread")
    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(jobs))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not failures, "; ".join(failures)
