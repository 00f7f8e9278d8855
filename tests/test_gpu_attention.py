"""Grouped-query decode attention on the GPU (moe_gqa_decode_attention through the C-ABI)
against the fp64 oracle, element by element.

Pages: MarkTechPost, "Perplexity open sources Lily, a Rust + Metal inference engine for
Qwen3.6-35B-A3B on Apple Silicon", body paragraphs 4 and 8.

Tolerance: the kernel keeps scores, the softmax and every sum in fp32 (the weights enter the
matrix cores as two bf16 pieces, about 2^-17 relative) and rounds the output to bf16, a
relative 2^-9; |got - ref| <= 8e-3 |ref| + 2e-3 rms(ref) leaves four times that margin.
"""
import numpy as np
import pytest

import oracle
from bit_grouped_expert_amd import _lib as L
from bit_grouped_expert_amd import device as dev
from bit_grouped_expert_amd import workload as wl

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    L.lib()
    return torch


def _run(torch, n_q, n_kv, ctx, stride=None, seed=0, q_scale=1.0):
    d = 128
    q, k, v = wl.make_attention_inputs(n_q, n_kv, d, ctx, stride, seed, q_scale)
    shp = L.gqa_shape(n_q, n_kv, d, ctx, stride)
    ws = torch.empty(L.moe_gqa_decode_workspace_bytes(shp), dtype=torch.uint8, device="cuda")
    out = torch.empty((n_q, d), dtype=torch.int16, device="cuda")
    L.moe_gqa_decode_attention(shp, dev.to_device(q), dev.to_device(k), dev.to_device(v), out, ws)
    torch.cuda.synchronize()
    got = wl.bf16_bits_to_f32(dev.to_host(out, np.uint16)).astype(np.float64)
    ref = oracle.gqa_decode_attention(q, k, v, ctx)
    return got, ref


def _check(got, ref, what):
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    rms = float(np.sqrt(np.mean(ref * ref)))
    err = np.abs(got - ref)
    bound = 8e-3 * np.abs(ref) + 2e-3 * rms
    bad = err > bound
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {bad.size} outside, worst "
                           f"{float((err - bound).max()):.3e} (rms {rms:.3e})")


@pytest.mark.parametrize("ctx", [1, 5, 127, 128, 129, 1000, 4096, 32768, 100000, 131072])
def test_attention_parity_ctx(torch_cuda, ctx):
    """16 query heads on two KV heads (the pages' layers), context from one position to 128K:
    a partial chunk, exact chunk multiples and one past, runs of several chunks per
    workgroup (a ragged last run at 100000), every output element."""
    say(f"gqa attention 16/2 ctx={ctx}")
    got, ref = _run(torch_cuda, 16, 2, ctx, seed=ctx)
    _check(got, ref, f"ctx {ctx}")


@pytest.mark.parametrize("n_q,n_kv", [(8, 8), (16, 1), (12, 3), (32, 2), (4, 4)])
def test_attention_parity_groups(torch_cuda, n_q, n_kv):
    """Group sizes 1 to 16 query heads per KV head (16 fills the matrix-core rows)."""
    say(f"gqa attention {n_q}/{n_kv} ctx=777")
    got, ref = _run(torch_cuda, n_q, n_kv, 777, seed=n_q * 10 + n_kv)
    _check(got, ref, f"{n_q}/{n_kv}")


def test_attention_stride_and_sharp_softmax(torch_cuda):
    """Caches allocated longer than ctx (NaN rows past it must never be read) and a query
    scaled by 8 (scores up to ~30: the per-chunk max keeps exp finite, and the chunks'
    maxima differ widely)."""
    say("gqa attention stride 5000 ctx 3001 q*8")
    got, ref = _run(torch_cuda, 16, 2, 3001, stride=5000, seed=7, q_scale=8.0)
    _check(got, ref, "stride, sharp")


def test_attention_repeatable(torch_cuda):
    """Two calls on the same inputs give the same bits (fixed reduction order)."""
    torch = torch_cuda
    d, ctx = 128, 2500
    q, k, v = wl.make_attention_inputs(16, 2, d, ctx, seed=3)
    shp = L.gqa_shape(16, 2, d, ctx)
    ws = torch.empty(L.moe_gqa_decode_workspace_bytes(shp), dtype=torch.uint8, device="cuda")
    qd, kd, vd = dev.to_device(q), dev.to_device(k), dev.to_device(v)
    outs = []
    for _ in range(2):
        out = torch.empty((16, d), dtype=torch.int16, device="cuda")
        L.moe_gqa_decode_attention(shp, qd, kd, vd, out, ws)
        outs.append(out)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])


def test_attention_sharp_softmax_long_runs(torch_cuda):
    """A query scaled by 8 over 40000 positions: each workgroup combines several chunks whose
    maxima differ widely, so the running maximum rises within a run and the sums are rescaled."""
    say("gqa attention ctx 40000 q*8")
    got, ref = _run(torch_cuda, 16, 2, 40000, seed=11, q_scale=8.0)
    _check(got, ref, "sharp, long runs")


def test_attention_graph_replay(torch_cuda):
    """Three calls (different queries and caches) captured into one HIP graph and replayed
    three times, with eager calls between the replays: every replay equals the eager result."""
    torch = torch_cuda
    d, ctx = 128, 9000
    shp = L.gqa_shape(16, 2, d, ctx)
    nbytes = L.moe_gqa_decode_workspace_bytes(shp)
    ins = []
    for s_ in range(3):
        q, k, v = wl.make_attention_inputs(16, 2, d, ctx, seed=20 + s_)
        ins.append((dev.to_device(q), dev.to_device(k), dev.to_device(v)))
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    outs = [torch.empty((16, d), dtype=torch.int16, device="cuda") for _ in range(3)]
    ref = []
    for (qd, kd, vd), o in zip(ins, outs):
        L.moe_gqa_decode_attention(shp, qd, kd, vd, o, ws)
        ref.append(o.clone())
    torch.cuda.synchronize()
    cur = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    side.wait_stream(cur)
    with torch.cuda.stream(side):
        for (qd, kd, vd), o in zip(ins, outs):
            L.moe_gqa_decode_attention(shp, qd, kd, vd, o, ws, stream=side)
    cur.wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cap = torch.cuda.current_stream()
        for (qd, kd, vd), o in zip(ins, outs):
            L.moe_gqa_decode_attention(shp, qd, kd, vd, o, ws, stream=cap)
    other = torch.empty((16, d), dtype=torch.int16, device="cuda")
    for rep in range(3):
        for o in outs:
            o.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        for i in range(3):
            assert torch.equal(outs[i], ref[i]), f"replay {rep}, call {i}"
        # eager work between the replays (it reuses the workspace)
        qd, kd, vd = ins[rep]
        L.moe_gqa_decode_attention(shp, qd, kd, vd, other, ws)
        torch.cuda.synchronize()
        assert torch.equal(other, ref[rep])
    del g
