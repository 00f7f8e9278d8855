"""Plain fp64 CPU oracle of grouped-query decode attention (one query token per call).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's CPU leg may
import this module.  The library's product path never calls it, and it shares no code
with the HIP kernels or their host layer.

Pages this follows (cited by title and section):
  [MTP] MarkTechPost, "Perplexity open sources Lily, a Rust + Metal inference engine for
        Qwen3.6-35B-A3B on Apple Silicon", body paragraph 4 (full-attention layers use
        grouped-query attention with 16 query heads and two KV heads, over a growing KV
        cache) and paragraph 8 (decode reads the key and value cache; several query heads
        share one KV head's rows, so each cached row is loaded once for all of them).
Readings taken where the pages are silent: head
dim 128 (d_model 2048 over 16 query heads); scaled dot-product attention, softmax over
q . k / sqrt(head dim), then the weighted sum of value rows; query head h reads KV head
h // (n_q / n_kv); the cache holds bf16 rows [KV head][position][head dim] and the query
is bf16; the one decode query attends to every cached position 0 .. ctx-1 (no further
mask); any rotary position encoding is already applied to the cached keys and the query.

Every quantity is float64 and nothing is rounded to bf16.  Each function is the definition
written out, with numpy dot products as the only library primitive.
"""
from __future__ import annotations

import numpy as np

from .moe_oracle import bf16_to_f64


def gqa_decode_attention(q_bits, k_bits, v_bits, ctx: int) -> np.ndarray:
    """[MTP] paras. 4 and 8.  q_bits bf16 [n_q, d]; k_bits, v_bits bf16 [n_kv, >= ctx, d].
    Returns the fp64 output [n_q, d]."""
    q = bf16_to_f64(q_bits)
    k = bf16_to_f64(np.asarray(k_bits)[:, :ctx])
    v = bf16_to_f64(np.asarray(v_bits)[:, :ctx])
    n_q, d = q.shape
    n_kv = k.shape[0]
    assert n_q % n_kv == 0 and ctx >= 1
    group = n_q // n_kv
    out = np.empty((n_q, d))
    for h in range(n_q):
        kv = h // group
        s = (k[kv] @ q[h]) / np.sqrt(d)     # one score per cached position
        p = np.exp(s - s.max())             # softmax numerators (shift-invariant)
        out[h] = (p @ v[kv]) / p.sum()
    return out
