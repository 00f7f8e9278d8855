"""Pins of the fp64 CPU oracle against facts that do not come from the oracle itself:
hand-worked values, exact integer arithmetic, brute force with exact rationals,
closed forms, invariants and a dense-MLP special case computed with torch.

Pages: MarkTechPost, "Perplexity open sources Lily, a Rust + Metal inference engine
for Qwen3.6-35B-A3B on Apple Silicon", body paragraphs 4-6; globalfeed.ai, "Perplexity
open sources Lily, a Rust and Metal inference engine for Apple Silicon", sections
"Requirements and model layout" and "Measurements".
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from bit_grouped_expert_amd import workload as wl

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _pack_py(codes):
    """Pure-Python packer written from the nibble-order reading (independent of workload.pack_codes)."""
    codes = list(codes)
    words = []
    for w in range(len(codes) // 8):
        v = 0
        for j in range(8):
            v |= (int(codes[8 * w + j]) & 15) << (4 * j)
        words.append(v)
    return np.array(words, dtype=np.uint32)


def _bf16(v):
    return wl.f32_to_bf16_bits(np.asarray(v, dtype=np.float32))


# ----------------------------------------------------------------------------- formats
def test_nibble_order_golden():
    g = _gold("nibble_order.json")
    words = np.array(g["words"], dtype=np.uint32)
    assert [int(w, 16) for w in g["words_hex"]] == g["words"]
    assert oracle.unpack_codes(words).tolist() == g["codes"]
    # the generator's packer and the test's packer agree with the hand words
    assert _pack_py(g["codes"]).tolist() == g["words"]
    assert wl.pack_codes(np.array(g["codes"])).tolist() == g["words"]


def test_bf16_widening_known_values():
    bits = np.array([0x3F80, 0xC000, 0x3F00, 0x0000, 0x8000, 0x4300, 0x7F7F], dtype=np.uint16)
    want = [1.0, -2.0, 0.5, 0.0, -0.0, 128.0, 3.3895313892515355e38]
    assert oracle.bf16_to_f64(bits).tolist() == want


def test_dequant_hand_example():
    g = _gold("dequant_hand.json")
    codes = [3] * 64 + [i % 16 for i in range(64)]
    words = _pack_py(codes)[None, :]
    scale = np.array([[int(h, 16) for h in g["scale_bf16"]]], dtype=np.uint16)
    bias = np.array([[int(h, 16) for h in g["bias_bf16"]]], dtype=np.uint16)
    W = oracle.dequantize(words, scale, bias)
    assert W.shape == (1, g["K"])
    assert np.all(W[0, :64] == g["expected_first_group_value"])
    assert W[0, 64:80].tolist() == g["expected_second_group_first16"]
    assert W[0, 80:96].tolist() == g["expected_second_group_first16"]


def test_format_matches_checkpoint_compression():
    """globalfeed.ai 'Requirements and model layout': about 70 GB of bf16 weights become 19.4 GB.
    4-bit codes plus one bf16 scale and one bf16 bias per 64 weights is 0.5625 B/weight,
    a 2/0.5625 = 3.56x ratio; the pages' 70/19.4 = 3.61x agrees within 2%.  (A g=32 or fp32
    scale/bias reading would give 3.2x and fail.)"""
    cfg = wl.MoEConfig("x", 0, 2048, 1, 1, 512)
    per_expert = wl.algorithmic_bytes(cfg, 1) - cfg.E * cfg.D * 4
    bytes_per_weight = per_expert / (3 * cfg.D * cfg.F)
    assert bytes_per_weight == 0.5625
    assert abs((2 / bytes_per_weight) / (70 / 19.4) - 1) < 0.02


# ----------------------------------------------------------------------------- exact integer GEMM
@pytest.mark.parametrize("epilogue", [0])
def test_grouped_gemm_exact_integer(epilogue):
    """scale = 1, bias = -8 gives w = q - 8, an integer; x in {-2..2}: the fp64 oracle must equal
    int64 matmul of the codes the test itself drew (no unpacking involved on this side)."""
    rng = np.random.default_rng(7)
    G, N, K = 3, 48, 192
    codes = rng.integers(0, 16, size=(G, N, K))
    words = np.stack([np.stack([_pack_py(codes[g, n]) for n in range(N)]) for g in range(G)])
    scale = np.full((G, N, K // 64), 0x3F80, dtype=np.uint16)
    bias = np.full((G, N, K // 64), 0xC100, dtype=np.uint16)    # -8.0
    counts = [5, 0, 11]
    off = np.concatenate([[0], np.cumsum(counts)])
    xi = rng.integers(-2, 3, size=(off[-1], K))
    C = oracle.grouped_gemm_q4(xi.astype(np.float64), off, words, scale, bias, epilogue)
    for g in range(G):
        want = xi[off[g]:off[g + 1]] @ (codes[g] - 8).T
        assert np.array_equal(C[off[g]:off[g + 1]], want.astype(np.float64))


def test_grouped_gemm_swiglu_integer_gate_up():
    """SwiGLU epilogue on an integer gate/up product: silu(g)*u with silu(z) = z/(1+e^-z)
    evaluated with math.exp per element."""
    rng = np.random.default_rng(8)
    N, K = 32, 64
    codes = rng.integers(0, 16, size=(1, N, K))
    words = np.stack([np.stack([_pack_py(codes[0, n]) for n in range(N)])])
    scale = np.full((1, N, 1), 0x3F80, dtype=np.uint16)
    bias = np.full((1, N, 1), 0xC100, dtype=np.uint16)
    xi = rng.integers(-2, 3, size=(4, K))
    C = oracle.grouped_gemm_q4(xi.astype(np.float64), [0, 4], words, scale, bias, 1)
    H = xi @ (codes[0] - 8).T
    for r in range(4):
        for f in range(N // 2):
            gte, up = float(H[r, f]), float(H[r, N // 2 + f])
            assert math.isclose(C[r, f], gte / (1 + math.exp(-gte)) * up, rel_tol=1e-14, abs_tol=1e-12)


# ----------------------------------------------------------------------------- routing
def test_routing_integer_ties_golden():
    g = _gold("routing_ties.json")
    E, D = 6, 64
    router = np.zeros((E, D), dtype=np.float32)
    router[:, 0] = g["router_column0"]
    router[:, 1] = g["router_column1"]
    x = np.zeros((3, D), dtype=np.float32)
    x[0, 0] = 1
    x[1, 1] = 1
    x[2, 0] = x[2, 1] = 1
    L = oracle.router_logits(_bf16(x), router)
    assert L[2].tolist() == [2, 5, 9, 5, 3, 6]
    idx3, w3 = oracle.select_topk(L, 3)
    idx1, w1 = oracle.select_topk(L, 1)
    assert idx3.tolist() == g["expected_top3"]
    assert idx1.tolist() == g["expected_top1"]
    assert np.allclose(w3[0], g["expected_weights_token0_top3"], rtol=0, atol=1e-15)
    assert np.all(w1 == 1.0)


def test_softmax_closed_form_and_invariants():
    """Softmax over the selected logits equals the full softmax renormalized over the top-k;
    with k = E it is the full softmax.  Weights sum to 1 and are non-increasing."""
    from scipy.special import softmax
    rng = np.random.default_rng(3)
    T, E, k = 64, 40, 8
    L = rng.standard_normal((T, E)) * 2
    idx, w = oracle.select_topk(L, k)
    full = softmax(L, axis=1)
    sel = np.take_along_axis(full, idx.astype(np.int64), axis=1)
    assert np.allclose(w, sel / sel.sum(1, keepdims=True), rtol=1e-13, atol=0)
    assert np.allclose(w.sum(1), 1.0, rtol=0, atol=1e-14)
    assert np.all(np.diff(w, axis=1) <= 0)
    # the selected set is exactly the k largest (brute force with Python sorting)
    for t in range(T):
        want = sorted(range(E), key=lambda e: (-L[t, e], e))[:k]
        assert idx[t].tolist() == want
    idxE, wE = oracle.select_topk(L, E)
    back = np.empty_like(wE)
    np.put_along_axis(back, idxE.astype(np.int64), wE, axis=1)
    assert np.allclose(back, full, rtol=1e-13, atol=0)


def test_histogram_scan_permutation_invariants():
    rng = np.random.default_rng(5)
    T, E, k = 300, 37, 5
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    idx[:40] = np.arange(k)            # a heavy group
    idx[:, 0][idx[:, 0] == 36] = 35    # keep expert 36 rare (maybe empty)
    idx = np.stack([row if len(set(row)) == k else np.arange(k) for row in idx])
    cnt = oracle.expert_histogram(idx, E)
    off, st, sr = oracle.stable_permutation(idx, E)
    assert cnt.sum() == T * k
    assert off[0] == 0 and off[-1] == T * k and np.all(np.diff(off) == cnt)
    assert np.array_equal(np.sort(sr), np.arange(T * k))          # bijection
    for t in range(T):
        for j in range(k):
            r = sr[t * k + j]
            assert st[r] == t
            e = idx[t, j]
            assert off[e] <= r < off[e + 1]
    for e in range(E):
        assert np.all(np.diff(st[off[e]:off[e + 1]]) > 0)          # ascending tokens in a group
    # brute force: sort the (expert, token) pairs with Python
    pairs = sorted((int(idx[t, j]), t) for t in range(T) for j in range(k))
    assert [p[1] for p in pairs] == st.tolist()


# ----------------------------------------------------------------------------- whole layer
def _tiny_weights(rng, G, D, F, scale_mag=0.05):
    def mat(N, K):
        codes = rng.integers(0, 16, size=(G, N, K))
        words = np.stack([np.stack([_pack_py(codes[g, n]) for n in range(N)]) for g in range(G)])
        s = _bf16(np.abs(rng.standard_normal((G, N, K // 64))) * scale_mag)
        b = _bf16(rng.standard_normal((G, N, K // 64)) * scale_mag)
        return codes, words, s, b
    c1, q1, s1, b1 = mat(2 * F, D)
    c2, q2, s2, b2 = mat(D, F)
    w = {"gate_up_q": q1, "gate_up_s": s1, "gate_up_b": b1, "down_q": q2, "down_s": s2, "down_b": b2}
    return w, (c1, s1, b1), (c2, s2, b2)


def _frac_bf16(bits):
    v = float(wl.bf16_bits_to_f32(np.uint16(bits)))
    return Fraction(v)


def test_brute_force_tiny_layer_exact_rationals():
    """The whole layer by pure-Python loops: exact rational logits and GEMMs, math.exp for the
    softmax and silu, the top-k by Python sort; against the numpy oracle to 1e-12."""
    rng = np.random.default_rng(11)
    T, D, E, k, F = 4, 64, 4, 2, 64
    x = _bf16(rng.standard_normal((T, D)))
    router = (rng.standard_normal((E, D)) * 0.3).astype(np.float32)
    weights, (c1, s1, b1), (c2, s2, b2) = _tiny_weights(rng, E + 1, D, F)
    res = oracle.moe_layer(x, router, weights, k)

    xf = [[_frac_bf16(x[t, d]) for d in range(D)] for t in range(T)]
    Rf = [[Fraction(float(router[e, d])) for d in range(D)] for e in range(E)]

    def wq(codes, s, b, g, n, c):
        return codes[g, n, c] * _frac_bf16(s[g, n, c // 64]) + _frac_bf16(b[g, n, c // 64])

    def ffn(g, xrow):
        h = [sum(xrow[c] * wq(c1, s1, b1, g, n, c) for c in range(D)) for n in range(2 * F)]
        a = [float(h[f]) / (1 + math.exp(-float(h[f]))) * float(h[F + f]) for f in range(F)]
        return [float(sum(Fraction(a[f]) * wq(c2, s2, b2, g, n, f) for f in range(F))) for n in range(D)]

    for t in range(T):
        logits = [sum(xf[t][d] * Rf[e][d] for d in range(D)) for e in range(E)]
        top = sorted(range(E), key=lambda e: (-logits[e], e))[:k]
        assert res["idx"][t].tolist() == top
        lmax = float(logits[top[0]])
        z = [math.exp(float(logits[e]) - lmax) for e in top]
        wts = [v / sum(z) for v in z]
        assert np.allclose(res["w"][t], wts, rtol=1e-13, atol=0)
        out = ffn(E, xf[t])
        for j, e in enumerate(top):
            y = ffn(e, xf[t])
            out = [o + wts[j] * yy for o, yy in zip(out, y)]
        scale = max(abs(v) for v in out)
        assert np.max(np.abs(res["out"][t] - np.array(out))) <= 1e-12 * scale


def test_dense_special_case_matches_torch():
    """One routed expert picked by every token (E = 1, k = 1, weight 1) plus the shared expert is
    two dense SwiGLU MLPs; compared with torch.nn.functional.silu and torch.matmul in fp64."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(12)
    T, D, F = 9, 128, 64
    x = _bf16(rng.standard_normal((T, D)))
    router = rng.standard_normal((1, D)).astype(np.float32)
    weights, (c1, s1, b1), (c2, s2, b2) = _tiny_weights(rng, 2, D, F)
    res = oracle.moe_layer(x, router, weights, 1)
    assert np.all(res["w"] == 1.0) and np.all(res["idx"] == 0)

    def tw(codes, s, b, g):
        c = torch.tensor(codes[g], dtype=torch.float64)
        sc = torch.tensor(wl.bf16_bits_to_f32(s[g]), dtype=torch.float64).repeat_interleave(64, dim=1)
        bi = torch.tensor(wl.bf16_bits_to_f32(b[g]), dtype=torch.float64).repeat_interleave(64, dim=1)
        return torch.addcmul(bi, c, sc)

    xt = torch.tensor(wl.bf16_bits_to_f32(x), dtype=torch.float64)
    out = torch.zeros(T, D, dtype=torch.float64)
    for g in (0, 1):
        h = torch.matmul(xt, tw(c1, s1, b1, g).t())
        a = torch.nn.functional.silu(h[:, :F]) * h[:, F:]
        out += torch.matmul(a, tw(c2, s2, b2, g).t())
    assert np.allclose(res["out"], out.numpy(), rtol=1e-12, atol=1e-12)


def test_zero_codes_give_shared_only():
    """Codes all 8 with bias = -8*scale give w = 0: routed experts contribute exactly 0 and
    the output equals the shared expert's output."""
    cfg = wl.MoEConfig("z", 8, 128, 4, 2, 64)
    x, router = wl.make_activations(cfg, 0)
    w = wl.make_weights(cfg, 1000)
    for key in ("gate_up", "down"):
        w[key + "_q"][:cfg.E] = 0x88888888
        s = oracle.bf16_to_f64(w[key + "_s"][:cfg.E])
        w[key + "_b"][:cfg.E] = wl.f32_to_bf16_bits((-8.0 * s).astype(np.float32))
    res = oracle.moe_layer(x, router, w, cfg.k)
    assert np.all(res["Y"] == 0)
    assert np.array_equal(res["out"], res["S"])
    res0 = oracle.moe_layer(x, router, w, cfg.k, with_shared=False)
    assert np.all(res0["out"] == 0)


def test_out_for_tokens_equals_layer_rows():
    cfg = wl.CONFIGS["tiny"]
    x, router = wl.make_activations(cfg, 0)
    w = wl.make_weights(cfg, 1000)
    full = oracle.moe_layer(x, router, w, cfg.k)
    toks = [0, 5, 6, 15]
    out, idx, wts = oracle.moe_out_for_tokens(x, router, w, cfg.k, toks)
    assert np.array_equal(idx, full["idx"][toks])
    assert np.allclose(out, full["out"][toks], rtol=1e-13, atol=1e-13)


def test_generator_recipe():
    cfg = wl.CONFIGS["tiny"]
    x, router = wl.make_activations(cfg, 0)
    w = wl.make_weights(cfg, 1000)
    assert x.shape == (16, 256) and x.dtype == np.uint16
    assert router.shape == (16, 256) and router.dtype == np.float32
    assert w["gate_up_q"].shape == (17, 256, 32) and w["gate_up_s"].shape == (17, 256, 4)
    assert w["down_q"].shape == (17, 256, 16) and w["down_s"].shape == (17, 256, 2)
    for key in ("gate_up", "down"):
        s = oracle.bf16_to_f64(w[key + "_s"])
        b = oracle.bf16_to_f64(w[key + "_b"])
        assert np.all(s >= 0)
        assert np.array_equal(b, -8 * s)  # the named workloads: bias = -8 * scale, exact
    wa = wl.make_weights(wl.CONFIGS["tiny_affine"], 1000)
    assert np.array_equal(wa["gate_up_q"], w["gate_up_q"])  # same codes and scales
    assert np.array_equal(wa["gate_up_s"], w["gate_up_s"])
    s = oracle.bf16_to_f64(wa["gate_up_s"])
    b = oracle.bf16_to_f64(wa["gate_up_b"])
    ratio = -b[s > 0] / s[s > 0]          # bias = -scale * (7.5 + 0.5 z), bf16-rounded
    assert abs(ratio.mean() - 7.5) < 0.05 and 0.4 < ratio.std() < 0.6
    assert not np.array_equal(b, -8 * s)
    codes = oracle.unpack_codes(w["down_q"])
    hist = np.bincount(codes.ravel(), minlength=16)
    assert hist.min() > 0.9 * codes.size / 16
    x2, _ = wl.make_activations(cfg, 0)
    assert np.array_equal(x, x2)


def test_zipf_routing_skew():
    """The skewed generator gives uneven groups including empty ones (small-T probe of the recipe)."""
    cfg = wl.MoEConfig("zipf_probe", 2048, 256, 64, 8, 64, routing="zipf")
    x, router = wl.make_activations(cfg, 0)
    L = oracle.router_logits(x, router)
    idx, _ = oracle.select_topk(L, cfg.k)
    cnt = oracle.expert_histogram(idx, cfg.E)
    assert np.all(cnt[-wl.ZIPF_MASKED:] == 0)
    assert cnt[0] > 4 * np.median(cnt)


# ----------------------------------------------------------------------------- decode attention
# MarkTechPost, same page, body paragraph 4 (grouped-query attention, 16 query heads and two
# KV heads) and paragraph 8 (decode over the KV cache).  bf16 bit patterns are written by hand
# here (exact small values), not through the library's generators.
def _bf(vals):
    """Exact bf16 bit patterns of float32 values that bf16 holds exactly."""
    a = np.asarray(vals, dtype=np.float32)
    u = a.view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "values must be exact in bf16"
    return (u >> 16).astype(np.uint16)


def test_attention_single_position_returns_its_value_row():
    """ctx = 1: softmax over one score is 1, so every head returns its KV head's value row; this
    also pins the head mapping h -> h // (n_q / n_kv)."""
    rng = np.random.default_rng(0)
    n_q, n_kv, d = 16, 2, 128
    q = _bf(rng.integers(-4, 5, (n_q, d)).astype(np.float32))
    k = _bf(rng.integers(-4, 5, (n_kv, 3, d)).astype(np.float32))
    v = _bf(rng.integers(-8, 9, (n_kv, 3, d)).astype(np.float32))
    out = oracle.gqa_decode_attention(q, k, v, 1)
    vf = v.astype(np.uint32) << 16
    vf = vf.view(np.float32).astype(np.float64)
    for h in range(n_q):
        assert np.array_equal(out[h], vf[h // 8, 0])


def test_attention_equal_keys_average_values():
    """All cached keys equal: every position gets the same weight, so the output is the mean of
    the value rows (exact rationals: small integers over ctx)."""
    rng = np.random.default_rng(1)
    n_q, n_kv, d, ctx = 4, 2, 128, 7
    q = _bf(rng.integers(-3, 4, (n_q, d)).astype(np.float32))
    krow = rng.integers(-3, 4, d).astype(np.float32)
    k = _bf(np.broadcast_to(krow, (n_kv, ctx, d)).copy())
    vint = rng.integers(-20, 21, (n_kv, ctx, d))
    v = _bf(vint.astype(np.float32))
    out = oracle.gqa_decode_attention(q, k, v, ctx)
    for h in range(n_q):
        exact = np.array([float(Fraction(int(vint[h // 2, :, j].sum()), ctx)) for j in range(d)])
        assert np.allclose(out[h], exact, rtol=0, atol=1e-12)


def test_attention_two_positions_hand_softmax():
    """Two positions with scores s0 = 2 * 8 / sqrt(128) and s1 = 0: weights e^s0 / (e^s0 + 1)
    and 1 / (e^s0 + 1), worked with math.exp.  Pins the 1 / sqrt(head dim) scale and the
    normalisation."""
    d = 128
    q = np.zeros((1, d), np.float32)
    q[0, 0] = 2.0
    k = np.zeros((1, 2, d), np.float32)
    k[0, 0, 0] = 8.0            # score 16 / sqrt(128)
    v = np.zeros((1, 2, d), np.float32)
    v[0, 0, :] = 1.0
    v[0, 1, :] = -3.0
    out = oracle.gqa_decode_attention(_bf(q), _bf(k), _bf(v), 2)
    s0 = 16.0 / math.sqrt(128.0)
    w0 = math.exp(s0) / (math.exp(s0) + 1.0)
    expect = w0 * 1.0 + (1.0 - w0) * (-3.0)
    assert abs(out[0, 0] - expect) < 1e-12 and abs(out[0, 5] - expect) < 1e-12


def test_attention_position_order_invariance_and_cache_tail():
    """Permuting the cached positions (keys with their values) leaves the output unchanged,
    and rows past ctx are never read."""
    rng = np.random.default_rng(3)
    n_q, n_kv, d, ctx = 16, 2, 128, 33
    q = wl.f32_to_bf16_bits(rng.standard_normal((n_q, d), dtype=np.float32))
    k = wl.f32_to_bf16_bits(rng.standard_normal((n_kv, ctx + 5, d), dtype=np.float32))
    v = wl.f32_to_bf16_bits(rng.standard_normal((n_kv, ctx + 5, d), dtype=np.float32))
    base = oracle.gqa_decode_attention(q, k, v, ctx)
    perm = rng.permutation(ctx)
    k2, v2 = k.copy(), v.copy()
    k2[:, :ctx] = k[:, perm]
    v2[:, :ctx] = v[:, perm]
    k2[:, ctx:] = 0x7FC0  # NaN rows past the cache length
    v2[:, ctx:] = 0x7FC0
    got = oracle.gqa_decode_attention(q, k2, v2, ctx)
    assert np.allclose(got, base, rtol=1e-12, atol=1e-12)
