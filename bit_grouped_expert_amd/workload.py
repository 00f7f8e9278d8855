"""Seeded synthetic inputs for the int4-g64 mixture-of-experts layer.

This module is shared by the CPU oracle's tests, the GPU parity tests and the
benchmark.  It draws random numbers, rounds them to bf16 bit patterns and
lays 4-bit codes out in the packed-word format the library consumes.  It holds
none of the layer's arithmetic (no dequantization, no routing, no GEMM).

Shapes follow the model layout described on the pages: 256 routed experts of
which the router picks 8, plus one shared expert that sees every token; expert
weights are groupwise-affine 4-bit with one bf16 scale and one bf16 bias per 64
weights.  Cited pages: the MarkTechPost report "Perplexity open sources Lily, a
Rust + Metal inference engine for Qwen3.6-35B-A3B on Apple Silicon" (body
paragraphs 4 and 5) and globalfeed.ai "Perplexity open sources Lily, a Rust and
Metal inference engine for Apple Silicon" (section "Requirements and model
layout").  The pages give no expert width; d_ff = 512 and d_model = 2048 are a
chosen Qwen3.6-35B-A3B-like shape.

Recipe (all numpy PCG64):
  activations, seed s:   x = bf16_rne(N(0,1)) [T, D];  R = fp32(N(0, 0.02)) [E, D]
  weights, seed s:       for each of gate_up (N=2F, K=D) then down (N=D, K=F),
                         over all G = E+1 groups at once (group E = shared expert):
                         codes: uniform random uint32 words [G, N, K/8], i.e. eight
                         independent uniform 4-bit codes per word;
                         scale = bf16_rne(|N(0, 0.02)|) [G, N, K/64];
                         bias, recipe "neg8" (the named workloads): bias = -8 * scale
                         (exact in bf16), so w = (q - 8) * scale;
                         bias, recipe "affine" (extra coverage): bias =
                         bf16_rne(-scale * (7.5 + 0.5 z)), z = N(0, 1) per group, drawn
                         after the scales (the bias of an affine 4-bit quantiser is the
                         group's minimum, near -7.5 scales for normal weights; drawn per
                         group, so it is not tied to the scale).
  skewed routing:        x[:, 0] = 1 and R[e, 0] = beta_e with
                         beta_e = -0.242 * ln(e+1) (Zipf-like popularity) and
                         beta_e = -1e4 for the last 4 experts (forced empty groups).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

GROUP = 64  # weights per (scale, bias) pair


@dataclass(frozen=True)
class MoEConfig:
    """One synthetic MoE-layer workload."""

    name: str
    T: int          # tokens
    D: int          # d_model
    E: int          # routed experts
    k: int          # experts picked per token
    F: int          # expert d_ff (SwiGLU)
    routing: str = "natural"   # "natural" (random router) or "zipf" (biased router)
    n_layers: int = 1          # distinct weight sets run back to back on the same x
    bias: str = "neg8"         # weight bias recipe: "neg8" (-8 * scale) or "affine"

    @property
    def G(self) -> int:
        """Weight groups including the shared expert."""
        return self.E + 1


CONFIGS = {
    # tiny layer: 16 tokens, d_model 256, 16 experts top-2 + shared, d_ff 128
    "tiny": MoEConfig("tiny", 16, 256, 16, 2, 128),
    # Qwen3.6-35B-A3B-shaped prefill of a 512-token prompt
    "prefill512": MoEConfig("prefill512", 512, 2048, 256, 8, 512),
    # batch-1 decode shapes
    "decode1": MoEConfig("decode1", 1, 2048, 256, 8, 512),
    "decode4": MoEConfig("decode4", 4, 2048, 256, 8, 512),
    # skewed-routing prefill (groups from 0 to ~2000 rows)
    "zipf8192": MoEConfig("zipf8192", 8192, 2048, 256, 8, 512, routing="zipf"),
    # same shape with natural (near-uniform) routing
    "uniform8192": MoEConfig("uniform8192", 8192, 2048, 256, 8, 512),
    # long-prompt chunk, four layers with distinct weights
    "long32768": MoEConfig("long32768", 32768, 2048, 256, 8, 512, n_layers=4),
    # the same shapes with a free per-group bias (extra coverage of the bias arithmetic)
    "tiny_affine": MoEConfig("tiny_affine", 16, 256, 16, 2, 128, bias="affine"),
    "prefill512_affine": MoEConfig("prefill512_affine", 512, 2048, 256, 8, 512, bias="affine"),
    "zipf8192_affine": MoEConfig("zipf8192_affine", 8192, 2048, 256, 8, 512, routing="zipf",
                                 bias="affine"),
}

ZIPF_S = 1.1
ZIPF_ALPHA = 0.22
ZIPF_MASKED = 4


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def f32_to_bf16_bits(a) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def pack_codes(codes) -> np.ndarray:
    """Pack 4-bit codes [..., K] (values 0..15) into uint32 words [..., K/8].

    Nibble j (bits 4j..4j+3) of word w holds the code of K index 8w + j.
    """
    c = np.asarray(codes, dtype=np.uint32)
    assert c.shape[-1] % 8 == 0
    c = c.reshape(c.shape[:-1] + (c.shape[-1] // 8, 8))
    out = np.zeros(c.shape[:-1], dtype=np.uint32)
    for j in range(8):
        out |= (c[..., j] & 0xF) << np.uint32(4 * j)
    return out


def zipf_bias(E: int) -> np.ndarray:
    """Router bias making expert popularity Zipf-like, with the last experts masked."""
    e = np.arange(E, dtype=np.float64)
    beta = -ZIPF_ALPHA * ZIPF_S * np.log(e + 1.0)
    beta[E - ZIPF_MASKED:] = -1.0e4
    return beta.astype(np.float32)


def make_activations(cfg: MoEConfig, seed: int = 0):
    """Return (x bf16 bits uint16[T, D], router fp32[E, D])."""
    rng = _rng(seed)
    x = f32_to_bf16_bits(rng.standard_normal((cfg.T, cfg.D), dtype=np.float32))
    router = (rng.standard_normal((cfg.E, cfg.D), dtype=np.float32) * np.float32(0.02))
    router = router.astype(np.float32)
    if cfg.routing == "zipf":
        x[:, 0] = f32_to_bf16_bits(np.float32(1.0))
        router[:, 0] = zipf_bias(cfg.E)
    return x, router


def _q4_matrix(rng, G, N, K, bias_recipe):
    assert K % GROUP == 0
    q = rng.integers(0, 2**32, size=(G, N, K // 8), dtype=np.uint32)
    s32 = np.abs(rng.standard_normal((G, N, K // GROUP), dtype=np.float32) * np.float32(0.02))
    scale = f32_to_bf16_bits(s32)
    if bias_recipe == "neg8":
        bias = f32_to_bf16_bits(np.float32(-8.0) * bf16_bits_to_f32(scale))
    elif bias_recipe == "affine":
        z = rng.standard_normal((G, N, K // GROUP), dtype=np.float32)
        bias = f32_to_bf16_bits(-bf16_bits_to_f32(scale) * (np.float32(7.5) + np.float32(0.5) * z))
    else:
        raise ValueError(f"unknown bias recipe {bias_recipe!r}")
    return q, scale, bias


def make_weights(cfg: MoEConfig, seed: int = 1000) -> dict:
    """Packed int4 weights for all E routed experts plus the shared expert (group E).

    gate_up: codes uint32[G, 2F, D/8], scale/bias bf16 bits uint16[G, 2F, D/64]
             (rows 0..F-1 are the gate projection, rows F..2F-1 the up projection)
    down:    codes uint32[G, D, F/8],  scale/bias uint16[G, D, F/64]
    """
    rng = _rng(seed)
    G, D, F = cfg.G, cfg.D, cfg.F
    w1q, w1s, w1b = _q4_matrix(rng, G, 2 * F, D, cfg.bias)
    w2q, w2s, w2b = _q4_matrix(rng, G, D, F, cfg.bias)
    return {
        "gate_up_q": w1q, "gate_up_s": w1s, "gate_up_b": w1b,
        "down_q": w2q, "down_s": w2s, "down_b": w2b,
    }


def layer_seed(layer: int) -> int:
    """Seed of the weight set of layer `layer`."""
    return 1000 + layer


def algorithmic_bytes(cfg: MoEConfig, touched_groups: int) -> int:
    """Bytes the layer must move at minimum: touched expert weights (4-bit codes plus one
    bf16 scale and one bf16 bias per 64 weights), the fp32 router, x in and out."""
    per_expert = 3 * cfg.D * cfg.F * (4 + 32 / GROUP) / 8
    return int(touched_groups * per_expert + cfg.E * cfg.D * 4 + 2 * cfg.T * cfg.D * 2)


def expert_flops(cfg: MoEConfig) -> int:
    """bf16 expert work: gate_up (2*D*2F) and down (2*F*D) per routed row, k+1 rows per token."""
    return 2 * 3 * cfg.D * cfg.F * (cfg.k + 1) * cfg.T


# ---- grouped-query decode attention inputs (the pages' full-attention layers: 16 query
# heads, two KV heads; head dim 128 is a reading).  Seeded, synthetic: q and the cached keys
# N(0, 1) (q scaled by q_scale to sharpen the softmax), values N(0, 1), all bf16; positions
# past ctx (up to kv_stride) hold `pad` (NaN by default, so that a read past the cache shows).
ATTN_CONFIGS = {
    # name: (n_q_heads, n_kv_heads, head_dim, ctx_len)
    "attn32k": (16, 2, 128, 32768),
    "attn4k": (16, 2, 128, 4096),
    "attn128k": (16, 2, 128, 131072),
}


def make_attention_inputs(n_q, n_kv, d, ctx, kv_stride=None, seed=0, q_scale=1.0, pad=0x7FC0):
    """Return (q bf16 bits [n_q, d], k bits [n_kv, kv_stride, d], v bits [n_kv, kv_stride, d])."""
    stride = ctx if kv_stride is None else kv_stride
    rng = _rng(seed)
    q = f32_to_bf16_bits(rng.standard_normal((n_q, d), dtype=np.float32) * np.float32(q_scale))
    k = np.full((n_kv, stride, d), pad, dtype=np.uint16)
    v = np.full((n_kv, stride, d), pad, dtype=np.uint16)
    k[:, :ctx] = f32_to_bf16_bits(rng.standard_normal((n_kv, ctx, d), dtype=np.float32))
    v[:, :ctx] = f32_to_bf16_bits(rng.standard_normal((n_kv, ctx, d), dtype=np.float32))
    return q, k, v


def attention_bytes(n_q, n_kv, d, ctx) -> int:
    """Algorithmic HBM bytes of one decode-attention call: the cached keys and values read once,
    the query read and the output written (bf16)."""
    return 2 * n_kv * ctx * d * 2 + 2 * n_q * d * 2
