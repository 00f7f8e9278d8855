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


@pytest.mark.parametrize("ctx", [1, 5, 127, 128, 129, 1000, 4096, 32768])
def test_attention_parity_ctx(torch_cuda, ctx):
    """16 query heads on two KV heads (the pages' layers), context from one position to 32K:
    a partial chunk, exact chunk multiples and one past, every output element."""
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
