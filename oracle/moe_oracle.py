"""Plain fp64 CPU oracle of the int4-g64 mixture-of-experts layer.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module.  The library's product path never
calls it, and it shares no code with the HIP kernels or their host layer.

Pages this follows (cited by title and section):
  [MTP] MarkTechPost, "Perplexity open sources Lily, a Rust + Metal inference
        engine for Qwen3.6-35B-A3B on Apple Silicon" (as carried in the
        aioga.com article record), body paragraphs 4-6.
  [GF]  globalfeed.ai, "Perplexity open sources Lily, a Rust and Metal
        inference engine for Apple Silicon", section "Requirements and model
        layout".
What the pages fix: a router scores 256 experts and picks 8, and one shared
expert sees every token ([MTP] para. 4, [GF] Requirements); expert weights are
groupwise-affine 4-bit with one bf16 scale and one bf16 bias per group of 64
([MTP] para. 5, [GF] Requirements); routed tokens form uneven per-expert groups
built by a histogram, a prefix scan and a scatter ([MTP] paras. 4 and 6).
Readings taken where the pages are silent (each also listed in the design
notes): affine dequant w = q*scale + bias with q unsigned 0..15; nibble j of a
packed word is K index 8w+j; a group is 64 consecutive input (K) indices;
weights are stored [N out, K in]; gate_up rows 0..F-1 are the gate and F..2F-1
the up projection; the expert FFN is SwiGLU, silu(z) = z / (1 + e^-z); routing
weights are a softmax over the selected k logits (equal to the full softmax
renormalized over the top-k); exact logit ties go to the lower expert id; the
permutation is stable (rows of one expert ascending in token id); the shared
expert has unit weight and the same d_ff; out = S + sum_j w_j * Y_j.

Every quantity is float64 (dequantized weights are exact in float64) and no
result is rounded to bf16.  There is no tiling, fusion or reordering: each
function is the definition, with numpy matmul as the only library primitive.
"""
from __future__ import annotations

import numpy as np

GROUP = 64


# --------------------------------------------------------------------------- formats
def bf16_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64; bf16 is the top half of an IEEE float32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def unpack_codes(words) -> np.ndarray:
    """Packed words uint32[..., K/8] -> 4-bit codes uint8[..., K].

    Reading: nibble j (bits 4j..4j+3) of word w is the code of K index 8w + j.
    """
    w = np.asarray(words, dtype=np.uint32)
    codes = np.empty(w.shape[:-1] + (w.shape[-1] * 8,), dtype=np.uint8)
    for j in range(8):
        codes[..., j::8] = (w >> np.uint32(4 * j)) & np.uint32(0xF)
    return codes


def dequantize(words, scale, bias) -> np.ndarray:
    """Groupwise affine 4-bit -> float64 weights [N, K]: w[n, c] = q[n, c]*s[n, c/64] + b[n, c/64].

    [MTP] para. 5 / [GF] Requirements: every group of 64 weights shares one bf16
    scale and one bf16 bias.
    """
    q = unpack_codes(words).astype(np.float64)
    s = np.repeat(bf16_to_f64(scale), GROUP, axis=-1)
    b = np.repeat(bf16_to_f64(bias), GROUP, axis=-1)
    assert q.shape == s.shape == b.shape, (q.shape, s.shape)
    return q * s + b


# --------------------------------------------------------------------------- routing
def router_logits(x_bits, router) -> np.ndarray:
    """L[t, e] = sum_d x[t, d] * R[e, d]; the router scores every expert ([MTP] para. 4)."""
    x = bf16_to_f64(x_bits)
    r = np.asarray(router, dtype=np.float32).astype(np.float64)
    return x @ r.T


def select_topk(logits, k: int):
    """Top-k experts per token by descending logit (exact ties: lower expert id first)
    and their routing weights softmax(L[t, idx]) over the k selected logits.

    [MTP] para. 4: the router picks 8 of 256.  The softmax-over-selected reading
    is an assumption (the pages do not state the weighting).
    """
    L = np.asarray(logits, dtype=np.float64)
    T, E = L.shape
    assert 1 <= k <= E
    order = np.argsort(-L, axis=1, kind="stable")  # stable: equal logits keep id order
    idx = order[:, :k].astype(np.int32)
    sel = np.take_along_axis(L, idx.astype(np.int64), axis=1)
    z = np.exp(sel - sel.max(axis=1, keepdims=True)) if T else sel
    w = z / z.sum(axis=1, keepdims=True) if T else sel
    return idx, w


def expert_histogram(idx, E: int) -> np.ndarray:
    """cnt[e] = number of (token, slot) pairs routed to expert e ([MTP] para. 6 "histogram")."""
    return np.bincount(np.asarray(idx, dtype=np.int64).ravel(), minlength=E).astype(np.int64)


def group_offsets(counts) -> np.ndarray:
    """Exclusive prefix sum: off[0] = 0, off[e+1] = off[e] + cnt[e] ([MTP] para. 6 "prefix scan")."""
    c = np.asarray(counts, dtype=np.int64)
    off = np.zeros(c.size + 1, dtype=np.int64)
    off[1:] = np.cumsum(c)
    return off


def stable_permutation(idx, E: int):
    """Scatter (token, slot) pairs into contiguous per-expert groups ([MTP] paras. 4 and 6).

    Returns (offsets[E+1], sorted_tok[T*k], slot_row[T*k]): the rows of expert e are
    off[e]..off[e+1]-1, holding its tokens in ascending token order; slot_row[t*k+j]
    is the row that pair (t, j) went to.  Written as a counting sort.
    """
    idx = np.asarray(idx, dtype=np.int64)
    T, k = idx.shape
    off = group_offsets(expert_histogram(idx, E))
    cursor = off[:-1].copy()
    sorted_tok = np.empty(T * k, dtype=np.int64)
    slot_row = np.empty(T * k, dtype=np.int64)
    for t in range(T):
        for j in range(k):
            e = idx[t, j]
            r = cursor[e]
            cursor[e] += 1
            sorted_tok[r] = t
            slot_row[t * k + j] = r
    return off, sorted_tok, slot_row


# --------------------------------------------------------------------------- expert FFN
def silu(z):
    return z / (1.0 + np.exp(-z))


def swiglu(h) -> np.ndarray:
    """[n, 2F] -> [n, F]: silu(gate) * up, gate = columns 0..F-1, up = F..2F-1."""
    F = h.shape[1] // 2
    return silu(h[:, :F]) * h[:, F:]


def grouped_gemm_q4(a_rows, offsets, words, scale, bias, epilogue: int = 0) -> np.ndarray:
    """C[r] = A[r] @ W_g^T for each row r of group g (rows off[g]..off[g+1]-1),
    W_g dequantized from group g's packed codes; epilogue 1 applies SwiGLU.

    a_rows: float64 [rows, K] (already gathered).  words: [G, N, K/8]; scale, bias: [G, N, K/64].
    """
    off = np.asarray(offsets, dtype=np.int64)
    G = off.size - 1
    N = words.shape[1]
    out_cols = N // 2 if epilogue == 1 else N
    C = np.zeros((off[-1], out_cols), dtype=np.float64)
    for g in range(G):
        r0, r1 = off[g], off[g + 1]
        if r1 == r0:
            continue
        W = dequantize(words[g], scale[g], bias[g])
        H = a_rows[r0:r1] @ W.T
        C[r0:r1] = swiglu(H) if epilogue == 1 else H
    return C


def expert_ffn(rows, w1, w2):
    """SwiGLU expert on float64 rows [n, D]: A = silu(x W1g^T) * (x W1u^T); Y = A W2^T."""
    A = swiglu(rows @ w1.T)
    return A, A @ w2.T


def combine(Y, slot_row, topk_w, S) -> np.ndarray:
    """out[t] = S[t] + sum_j w[t, j] * Y[slot_row[t*k + j]] (S = shared expert, unit weight)."""
    w = np.asarray(topk_w, dtype=np.float64)
    T, k = w.shape
    rows = np.asarray(slot_row, dtype=np.int64).reshape(T, k)
    out = np.array(S, dtype=np.float64, copy=True)
    for j in range(k):
        out += w[:, j:j + 1] * Y[rows[:, j]]
    return out


# --------------------------------------------------------------------------- whole layer
def _ffn_weights(weights, g):
    w1 = dequantize(weights["gate_up_q"][g], weights["gate_up_s"][g], weights["gate_up_b"][g])
    w2 = dequantize(weights["down_q"][g], weights["down_s"][g], weights["down_b"][g])
    return w1, w2


def moe_layer(x_bits, router, weights, k: int, with_shared: bool = True) -> dict:
    """The whole layer, every intermediate kept (float64).

    weights: dict of gate_up_{q,s,b} [G, 2F, D/8 | D/64] and down_{q,s,b} [G, D, F/8 | F/64];
    groups 0..E-1 are the routed experts, group E (if with_shared) the shared expert.
    """
    x = bf16_to_f64(x_bits)
    T, D = x.shape
    E = np.asarray(router).shape[0]
    F = weights["down_q"].shape[2] * 8
    L = router_logits(x_bits, router)
    idx, w = select_topk(L, k)
    off, sorted_tok, slot_row = stable_permutation(idx, E)
    A = np.zeros((T * k, F))
    Y = np.zeros((T * k, D))
    for e in range(E):
        r0, r1 = off[e], off[e + 1]
        if r1 == r0:
            continue
        w1, w2 = _ffn_weights(weights, e)
        A[r0:r1], Y[r0:r1] = expert_ffn(x[sorted_tok[r0:r1]], w1, w2)
    if with_shared:
        w1, w2 = _ffn_weights(weights, E)
        A_s, S = expert_ffn(x, w1, w2)
    else:
        A_s, S = np.zeros((T, F)), np.zeros((T, D))
    out = combine(Y, slot_row, w, S)
    return {"logits": L, "idx": idx, "w": w, "counts": np.diff(off), "offsets": off,
            "sorted_tok": sorted_tok, "slot_row": slot_row, "A": A, "Y": Y,
            "A_shared": A_s, "S": S, "out": out}


def moe_out_for_tokens(x_bits, router, weights, k: int, tokens, with_shared: bool = True):
    """The layer's output rows for a subset of tokens (float64 [len(tokens), D]).

    Routing and the expert FFN act on each token alone, so out[t] depends only on
    x[t]: this is the same definition evaluated on the selected rows.
    Returns (out_rows, idx_rows, w_rows).
    """
    tokens = np.asarray(tokens, dtype=np.int64)
    xs = np.asarray(x_bits)[tokens]
    E = np.asarray(router).shape[0]
    L = router_logits(xs, router)
    idx, w = select_topk(L, k)
    x = bf16_to_f64(xs)
    out = np.zeros_like(x)
    for e in np.unique(idx):
        sel_t, sel_j = np.nonzero(idx == e)
        w1, w2 = _ffn_weights(weights, int(e))
        _, y = expert_ffn(x[sel_t], w1, w2)
        out[sel_t] += w[sel_t, sel_j][:, None] * y
    if with_shared:
        w1, w2 = _ffn_weights(weights, E)
        out += expert_ffn(x, w1, w2)[1]
    return out, idx, w
