"""GPU parity of the HIP path (called through the C ABI) against the fp64 CPU oracle.

Bars: integer work (top-k indices in order, group offsets, permutation) bit-exact; grouped
GEMM on exact-integer weights bit-exact after bf16 rounding; bf16 outputs per element within
|gpu - oracle| <= 2e-2 * RMS(oracle) + 3e-2 * |oracle| (the reading of the stated tolerance,
derived from the bf16 rounding points of the path).
"""
import math
import sys

import numpy as np
import pytest

import oracle
from bit_grouped_expert_amd import _lib as L
from bit_grouped_expert_amd import device as dev
from bit_grouped_expert_amd import workload as wl

pytestmark = pytest.mark.gpu

ATOL_RMS, RTOL = 2e-2, 3e-2
WSUM_TOL = 8 * 2.0 ** -23   # |sum_j w_tj - 1|: eight fp32 roundings of a quotient and a sum

ENGINES = ["grouped", "resident", "wide"]


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    L.lib()
    return torch


def bf16f(bits):
    return oracle.bf16_to_f64(bits)


def check_tol(g, o, what):
    g = np.asarray(g, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    rms = math.sqrt(float(np.mean(o * o))) if o.size else 0.0
    err = np.abs(g - o)
    bound = ATOL_RMS * rms + RTOL * np.abs(o)
    bad = err > bound
    say(f"  {what}: max|err|/RMS = {err.max() / rms if rms else 0:.4g}, "
        f"mean|err|/RMS = {err.mean() / rms if rms else 0:.3g}, "
        f"failing = {int(bad.sum())}/{err.size}")
    assert not bad.any(), f"{what}: {int(bad.sum())} elements outside tolerance"


def call_or_skip(fn, *a, **kw):
    """Run an entry point with a forced engine; skip when that engine cannot take the shape."""
    try:
        fn(*a, **kw)
    except L.MoEError as e:
        if e.status == L.MOE_ERR_SHAPE:
            pytest.skip("the forced engine cannot take this shape")
        raise


# ----------------------------------------------------------------------------- grouped GEMM
def _q4_codes_words(rng, G, N, K):
    codes = rng.integers(0, 16, size=(G, N, K), dtype=np.uint8)
    return codes, wl.pack_codes(codes)


GEMM_INT_CASES = [
    # (counts per group, N, K, gather)
    ([0, 1, 17, 33, 100], 128, 256, False),
    ([64, 5, 40], 64, 64, False),            # K = 64: only a trailing half block
    ([16, 0, 31, 70], 192, 192, True),       # 128 + 64, gathered rows incl. invalid indices
    ([200, 30], 256, 2048, True),            # 64-row tiles, every fragment count
    ([3, 0, 0, 9], 512, 512, False),
    ([127, 128, 129, 0, 300, 1], 384, 320, True),   # 128-row tiles: full, ragged, partial waves
    ([127, 128, 129, 0, 300, 1], 384, 384, True),   # K % 128 == 0
    ([5, 0, 70, 3], 320, 128, True),                # one 128-K stage per item
    ([0, 1, 17, 33, 100], 256, 1024, True),         # two halves of K, two 256-K stages each
    ([40, 0, 129, 300], 256, 256, True),            # one 256-K stage: four groups in every bias form
    ([5, 0, 70, 3, 16], 512, 1536, False),          # halves of three stages, no prefetch
    ([1, 31, 32, 33], 768, 256, False),             # one stage over the whole K
    ([40, 2, 0, 27], 256, 512, True),               # whole K per wavefront, two stages
    ([257, 0, 600, 1, 130], 256, 256, True),        # 128-row tiles: full, 1-row, ragged
    ([513, 16, 255], 512, 512, False),              # two weight blocks of 256 rows
    ([300, 129], 768, 768, True),                   # three weight blocks, twelve 64-K stages
]


def _int_gemm_inputs(case, bias_val, seed_base=100):
    counts, N, K, gather = GEMM_INT_CASES[case] if isinstance(case, int) else case
    rng = np.random.default_rng(seed_base + (case if isinstance(case, int) else 0))
    G = len(counts)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    rows = int(off[-1])
    codes, words = _q4_codes_words(rng, G, N, K)
    scale = np.full((G, N, K // 64), 0x3F80, np.uint16)
    bias = np.full((G, N, K // 64), wl.f32_to_bf16_bits(np.float32(bias_val)), np.uint16)
    a_rows = rows + 7
    xi = rng.integers(-2, 3, size=(a_rows, K))
    A = wl.f32_to_bf16_bits(xi.astype(np.float32))
    if gather:
        ridx = rng.integers(0, a_rows, size=rows).astype(np.int32)
        ridx[::11] = -1
        ridx[5::13] = a_rows          # out of range -> zero row
    else:
        ridx = None
    gathered = np.zeros((rows, K))
    src = ridx if gather else np.arange(rows)
    ok = (src >= 0) & (src < a_rows)
    gathered[ok] = bf16f(A[src[ok]])
    return G, N, K, off, rows, words, scale, bias, A, a_rows, ridx, gathered


def _run_gemm(torch, G, rows, N, K, A, a_rows, ridx, off, words, scale, bias, epilogue, engine):
    d = dev.to_device
    out_cols = N // 2 if epilogue else N
    Cdev = torch.full((rows, out_cols), 0x7FC1, dtype=torch.int16, device="cuda")
    ws = torch.empty(L.moe_grouped_gemm_q4_workspace_bytes(G, rows, a_rows, K), dtype=torch.uint8,
                     device="cuda")
    tw = [d(words), d(scale), d(bias)]
    keep = [d(A), d(ridx) if ridx is not None else None, d(off)]
    call_or_skip(L.moe_grouped_gemm_q4_ex, G, rows, N, K, keep[0], a_rows, keep[1], keep[2],
                 L.q4(*tw), epilogue, Cdev, ws, engine)
    torch.cuda.synchronize()
    return dev.to_host(Cdev, np.uint16)


@pytest.mark.parametrize("engine", ENGINES)
@pytest.mark.parametrize("bias_val", [-8, -5])
@pytest.mark.parametrize("case", range(len(GEMM_INT_CASES)))
def test_grouped_gemm_exact_integer(torch_cuda, case, bias_val, engine):
    """scale 1, bias -8 or -5 (w = q - 8 or q - 5), x in {-2..2}: every partial sum is an
    integer below 2^24, so the bf16-rounded GPU output must equal the bf16 rounding of the
    exact result bit for bit.  Bias -5 exercises the path for b != -8 s."""
    G, N, K, off, rows, words, scale, bias, A, a_rows, ridx, gathered = \
        _int_gemm_inputs(case, bias_val)
    say(f"int gemm case {case} [{engine}] bias {bias_val}: counts={np.diff(off).tolist()} "
        f"N={N} K={K}")
    ref = oracle.grouped_gemm_q4(gathered, off, words, scale, bias, 0)
    assert np.array_equal(ref, np.round(ref))
    want = wl.f32_to_bf16_bits(ref.astype(np.float32))
    got = _run_gemm(torch_cuda, G, rows, N, K, A, a_rows, ridx, off, words, scale, bias, 0, engine)
    assert np.array_equal(got, want), f"{int((got != want).sum())} mismatching elements"


SWIGLU_INT_CASES = [
    ([0, 3, 17, 40, 129], 64, 256, True),     # F = 32: a partial slice of every engine's block
    ([33, 0, 200, 5], 192, 512, False),       # F = 96
    ([1, 64, 16, 130], 384, 1024, True),      # F = 192
    ([20, 0, 300], 1024, 2048, True),         # F = 512, the layer's gate_up shape
    ([9, 70, 1], 256, 768, False),            # F = 128, three stages
]


@pytest.mark.parametrize("engine", ENGINES)
@pytest.mark.parametrize("case", range(len(SWIGLU_INT_CASES)))
def test_grouped_gemm_integer_swiglu(torch_cuda, case, engine):
    """The SwiGLU epilogue on exact integer products (scale 1, bias -8, x in {-2..2}): H is
    exact in fp32, so the output differs from the oracle's silu(H_g) * H_u only by the fp32
    evaluation of silu and the final bf16 rounding."""
    G, N, K, off, rows, words, scale, bias, A, a_rows, ridx, gathered = \
        _int_gemm_inputs(SWIGLU_INT_CASES[case], -8, seed_base=300 + case)
    say(f"int swiglu case {case} [{engine}]: counts={np.diff(off).tolist()} N={N} K={K}")
    ref = oracle.grouped_gemm_q4(gathered, off, words, scale, bias, 1)
    got = _run_gemm(torch_cuda, G, rows, N, K, A, a_rows, ridx, off, words, scale, bias, 1, engine)
    check_tol(bf16f(got), ref, f"integer swiglu case {case} [{engine}]")


@pytest.mark.parametrize("engine", ENGINES)
@pytest.mark.parametrize("bias", ["neg8", "affine", "free"])
@pytest.mark.parametrize("epilogue", [0, 1])
@pytest.mark.parametrize("counts", [[0, 3, 16, 29, 64, 90, 1], [250, 0, 131, 7, 384]])
@pytest.mark.parametrize("K", [1024, 768, 512])
def test_grouped_gemm_float_vs_oracle(torch_cuda, K, epilogue, counts, bias, engine):
    """Float weights with the generator's bias recipes (-8 scale; -scale (7.5 + 0.5 z) per
    group) and, with "free", biases drawn independently of the scale and of either sign.
    K = 1024, 768 and 512 take the three ways the wide-tile engine forms the bias term
    (once per block over 32 groups, per stage, once per block with the pieces of X side by
    side)."""
    torch = torch_cuda
    rng = np.random.default_rng(7 + epilogue)
    say(f"float gemm [{engine}] K={K} epilogue={epilogue} counts={counts} bias={bias}")
    G, N = len(counts), 256
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    rows = int(off[-1])
    cfg = wl.MoEConfig("g", 0, K, G - 1, 1, N // 2, bias="neg8" if bias == "neg8" else "affine")
    w = wl.make_weights(cfg, 1234 + epilogue)      # gate_up: [G, N, K/8]
    words, scale, bvals = w["gate_up_q"], w["gate_up_s"], w["gate_up_b"]
    if bias == "free":
        bvals = wl.f32_to_bf16_bits(rng.standard_normal(bvals.shape).astype(np.float32) * 0.1)
    A = wl.f32_to_bf16_bits(rng.standard_normal((rows, K)).astype(np.float32))
    ref = oracle.grouped_gemm_q4(bf16f(A), off, words, scale, bvals, epilogue)
    got = _run_gemm(torch, G, rows, N, K, A, rows, None, off, words, scale, bvals, epilogue, engine)
    check_tol(bf16f(got), ref, f"grouped gemm epilogue={epilogue}")


# ----------------------------------------------------------------------------- routing
ROUTE_CONFIGS = ["tiny", "decode1", "decode4", "prefill512", "zipf8192", "uniform8192", "long32768"]


def _route_gpu(torch, cfg, x, router, gap=None):
    shp = L.shape(cfg.T, cfg.D, cfg.E, cfg.k, cfg.F)
    ws = dev.workspace(shp)
    idx = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device="cuda")
    w = torch.empty((cfg.T, cfg.k), dtype=torch.float32, device="cuda")
    xd, rd = dev.to_device(x), dev.to_device(router)
    if gap is None:
        L.moe_route(shp, xd, rd, idx, w, ws)
    else:
        L.moe_route_ex(shp, xd, rd, idx, w, gap, ws)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), w.cpu().numpy()


def _check_route(cfg, x, router, gi, gw):
    """Ordered top-k equal to the oracle's fp64 order (ties: lower id), weights per
    (token, slot) within 2e-5, and every token's weights summing to 1 within 8 * 2^-23."""
    Lref = oracle.router_logits(x, router)
    ri, rw = oracle.select_topk(Lref, cfg.k)
    same_set = np.all(np.sort(gi, 1) == np.sort(ri, 1), axis=1)
    if not same_set.all():
        s = np.sort(Lref, 1)[:, ::-1]
        bad = np.nonzero(~same_set)[0]
        say("  mismatching tokens", bad[:10], "fp64 gaps", (s[bad, cfg.k - 1] - s[bad, cfg.k])[:10])
    assert same_set.all(), f"{int((~same_set).sum())} tokens with a different top-{cfg.k} set"
    same_order = np.all(gi == ri, axis=1)
    assert same_order.all(), \
        f"{int((~same_order).sum())} tokens with the top-{cfg.k} set in another order"
    assert np.max(np.abs(gw - rw)) < 2e-5, np.max(np.abs(gw - rw))
    wsum = gw.astype(np.float64).sum(1)
    assert np.max(np.abs(wsum - 1.0)) <= WSUM_TOL, np.max(np.abs(wsum - 1.0))
    # weights come from the fp32 logits, so within a run of fp32-close logits that the exact
    # order rearranged they may rise by a rounding error
    assert np.all(np.diff(gw.astype(np.float64), axis=1) <= 1e-6), "weights not descending"


@pytest.mark.parametrize("name", ROUTE_CONFIGS)
def test_route_parity(torch_cuda, name):
    cfg = wl.CONFIGS[name]
    say(f"route {name}: T={cfg.T} E={cfg.E} k={cfg.k}")
    x, router = wl.make_activations(cfg, 0)
    gi, gw = _route_gpu(torch_cuda, cfg, x, router)
    _check_route(cfg, x, router, gi, gw)


def test_route_forced_refine(torch_cuda):
    """Every token through the exact fp64 rescoring: the order equals the fp64 order too."""
    cfg = wl.CONFIGS["prefill512"]
    x, router = wl.make_activations(cfg, 0)
    gi, gw = _route_gpu(torch_cuda, cfg, x, router, gap=1e30)
    _check_route(cfg, x, router, gi, gw)


def test_route_close_logits_inside_selection(torch_cuda):
    """Selected experts whose logits differ by less than the fp32 error: router rows that
    differ from a base row only by tiny multiples of one feature, so many selected logits are
    within 1e-6 of each other; the order must still be the exact fp64 order."""
    rng = np.random.default_rng(11)
    cfg = wl.MoEConfig("close", 96, 256, 64, 8, 64)
    x = wl.f32_to_bf16_bits(rng.standard_normal((cfg.T, cfg.D)).astype(np.float32))
    base = (rng.standard_normal((8, cfg.D)) * 0.02).astype(np.float32)
    router = base[rng.integers(0, 8, size=cfg.E)].copy()
    router[:, 5] += (np.arange(cfg.E) % 7 * 3e-7).astype(np.float32)
    gi, gw = _route_gpu(torch_cuda, cfg, x, router)
    _check_route(cfg, x, router, gi, gw)


@pytest.mark.parametrize("E,k,T,D", [(64, 8, 64, 128), (1000, 4, 40, 64), (40, 32, 33, 128)])
def test_route_exact_ties(torch_cuda, E, k, T, D):
    """Integer x and router rows (many duplicated) give exactly tied logits: the lower expert id
    wins and the order is the exact descending order."""
    rng = np.random.default_rng(E + k)
    cfg = wl.MoEConfig("ties", T, D, E, k, 64)
    x = wl.f32_to_bf16_bits(rng.integers(-2, 3, size=(T, D)).astype(np.float32))
    base = rng.integers(-3, 4, size=(max(E // 4, 2), D)).astype(np.float32)
    router = base[rng.integers(0, base.shape[0], size=E)]
    gi, gw = _route_gpu(torch_cuda, cfg, x, router)
    _check_route(cfg, x, router, gi, gw)


@pytest.mark.parametrize("T,D,E,k", [(2500, 192, 40, 4), (2100, 512, 200, 6), (2050, 256, 300, 5)])
def test_route_many_tokens_off_shapes(torch_cuda, T, D, E, k):
    """The many-token routers away from the layer's shape: d_model not a multiple of 256 (R
    split once into bf16 planes, 64-token tiles of 32 experts), and multiples of 256 (the
    64 x 128 tile kernel) with expert counts that leave a partial expert tile (up to 300
    experts: the top-k's widest form) and token counts that leave a partial token tile."""
    cfg = wl.MoEConfig("route_many", T, D, E, k, 64)
    say(f"route T={T} D={D} E={E} k={k}")
    x, router = wl.make_activations(cfg, 3)
    gi, gw = _route_gpu(torch_cuda, cfg, x, router)
    _check_route(cfg, x, router, gi, gw)


# ----------------------------------------------------------------------------- permutation
def _permute_gpu(torch, cfg, idx):
    shp = L.shape(cfg.T, cfg.D, cfg.E, cfg.k, cfg.F)
    ws = dev.workspace(shp)
    n = max(cfg.T * cfg.k, 1)
    off = torch.empty(cfg.E + 1, dtype=torch.int32, device="cuda")
    st = torch.full((n,), -7, dtype=torch.int32, device="cuda")
    sr = torch.full((n,), -7, dtype=torch.int32, device="cuda")
    idx_d = dev.to_device(idx.astype(np.int32))
    L.moe_permute(shp, idx_d, off, st, sr, ws)
    torch.cuda.synchronize()
    return off.cpu().numpy(), st.cpu().numpy(), sr.cpu().numpy()


@pytest.mark.parametrize("name", ["tiny", "decode1", "prefill512", "zipf8192", "long32768"])
def test_permute_parity(torch_cuda, name):
    cfg = wl.CONFIGS[name]
    say(f"permute {name}")
    x, router = wl.make_activations(cfg, 0)
    idx, _ = oracle.select_topk(oracle.router_logits(x, router), cfg.k)
    off, st, sr = _permute_gpu(torch_cuda, cfg, idx)
    r_off, r_st, r_sr = oracle.stable_permutation(idx, cfg.E)
    assert np.array_equal(off, r_off)
    assert np.array_equal(st, r_st)
    assert np.array_equal(sr, r_sr)


@pytest.mark.parametrize("T,E,k", [(2100, 300, 6), (1000, 1000, 4), (3000, 17, 3), (257, 257, 32)])
def test_permute_off_shapes(torch_cuda, T, E, k):
    """The standalone permutation's two forms away from the layer's shape (one workgroup per
    four experts up to 8192 pairs and 1024 experts, count / scan / scatter beyond), on
    seeded distinct expert ids per token, top_k up to 32: offsets, permuted tokens and rows
    bit-exact."""
    cfg = wl.MoEConfig("perm_off", T, 64, E, k, 64)
    say(f"permute T={T} E={E} k={k}")
    rng = np.random.default_rng(T + E + k)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    off, st, sr = _permute_gpu(torch_cuda, cfg, idx)
    r_off, r_st, r_sr = oracle.stable_permutation(idx, E)
    assert np.array_equal(off, r_off)
    assert np.array_equal(st, r_st)
    assert np.array_equal(sr, r_sr)


def test_permute_invalid_entries_and_empty(torch_cuda):
    """Entries outside [0, E) are ignored: they behave like an extra expert after the last
    one that is then dropped, and their slot_row is -1."""
    cfg = wl.MoEConfig("inv", 700, 64, 30, 3, 64)
    rng = np.random.default_rng(3)
    idx = np.stack([rng.permutation(cfg.E)[:cfg.k] for _ in range(cfg.T)]).astype(np.int32)
    idx[::17, 1] = -1
    idx[5::23, 2] = cfg.E
    off, st, sr = _permute_gpu(torch_cuda, cfg, idx)
    mapped = np.where((idx < 0) | (idx >= cfg.E), cfg.E, idx)
    r_off, r_st, r_sr = oracle.stable_permutation(mapped, cfg.E + 1)
    valid = (idx.ravel() >= 0) & (idx.ravel() < cfg.E)
    assert np.array_equal(off, r_off[:cfg.E + 1])
    n = r_off[cfg.E]
    assert np.array_equal(st[:n], r_st[:n])
    assert np.array_equal(sr[valid], r_sr[valid])
    assert np.all(sr[~valid] == -1)
    # T = 0: offsets all zero
    cfg0 = wl.MoEConfig("empty", 0, 64, 30, 3, 64)
    off0, _, _ = _permute_gpu(torch_cuda, cfg0, np.zeros((0, 3), np.int32))
    assert np.all(off0 == 0)


# ----------------------------------------------------------------------------- combine
@pytest.mark.parametrize("with_shared", [True, False])
def test_combine_parity(torch_cuda, with_shared):
    torch = torch_cuda
    cfg = wl.MoEConfig("c", 300, 2048 + 64, 32, 5, 64)
    T, D, k = cfg.T, cfg.D, cfg.k
    rng = np.random.default_rng(9)
    Y = wl.f32_to_bf16_bits(rng.standard_normal((T * k, D)).astype(np.float32))
    S = wl.f32_to_bf16_bits(rng.standard_normal((T, D)).astype(np.float32))
    w = rng.random((T, k)).astype(np.float32)
    sr = rng.permutation(T * k).astype(np.int32)
    sr[::19] = -1
    sr[7::31] = T * k
    out = torch.empty((T, D), dtype=torch.int16, device="cuda")
    keep = [dev.to_device(Y), dev.to_device(sr), dev.to_device(w), dev.to_device(S)]
    L.moe_combine(L.shape(T, D, cfg.E, k, cfg.F), keep[0], keep[1], keep[2],
                  keep[3] if with_shared else None, out)
    torch.cuda.synchronize()
    valid = (sr >= 0) & (sr < T * k)
    w_eff = np.where(valid.reshape(T, k), w, 0.0)
    ref = oracle.combine(bf16f(Y), np.where(valid, sr, 0), w_eff,
                         bf16f(S) if with_shared else np.zeros((T, D)))
    check_tol(bf16f(dev.to_host(out, np.uint16)), ref, "combine")


# ----------------------------------------------------------------------------- whole layer
def _layer_gpu(torch, cfg, x, router, lw, with_shared=True, engine="auto"):
    shp = L.shape(cfg.T, cfg.D, cfg.E, cfg.k, cfg.F)
    ws = dev.workspace(shp)
    out = torch.empty((cfg.T, cfg.D), dtype=torch.int16, device="cuda")
    xd, rd = dev.to_device(x), dev.to_device(router)
    call_or_skip(L.moe_layer_forward_ex, shp, xd, rd, lw.experts,
                 lw.shared if with_shared else None, out, ws, L.layer_opts(engine))
    torch.cuda.synchronize()
    lay = L.moe_workspace_layout(shp)
    wsn = ws.cpu().numpy()
    del ws

    def grab(off, count, dtype):
        return wsn[off:off + count * np.dtype(dtype).itemsize].view(dtype).copy()
    inter = {
        "idx": grab(lay.topk_idx, cfg.T * cfg.k, np.int32).reshape(cfg.T, cfg.k),
        "w": grab(lay.topk_w, cfg.T * cfg.k, np.float32).reshape(cfg.T, cfg.k),
        "offsets": grab(lay.offsets, cfg.E + 2, np.int32),
        "sorted_tok": grab(lay.sorted_tok, (cfg.k + 1) * cfg.T, np.int32),
        "slot_row": grab(lay.slot_row, cfg.T * cfg.k, np.int32),
    }
    # the persistent launches' waits all ended before their bound
    assert grab(lay.sync, 1, np.int32)[0] == 0
    return dev.to_host(out, np.uint16), inter


def _check_layer_integer_stages(cfg, x, router, inter, with_shared=True):
    """Ordered top-k and the permutation equal the oracle's own, on every token."""
    idx = inter["idx"]
    ri, _ = oracle.select_topk(oracle.router_logits(x, router), cfg.k)
    assert np.array_equal(idx, ri), f"{int((idx != ri).any(1).sum())} tokens with another top-k"
    r_off, r_st, r_sr = oracle.stable_permutation(ri, cfg.E)
    assert np.array_equal(inter["offsets"][:cfg.E + 1], r_off)
    n = cfg.T * cfg.k
    assert np.array_equal(inter["sorted_tok"][:n], r_st)
    assert np.array_equal(inter["slot_row"], r_sr)
    if with_shared:
        assert inter["offsets"][cfg.E + 1] == n + cfg.T
        assert np.array_equal(inter["sorted_tok"][n:], np.arange(cfg.T))


def _layer_full_check(torch_cuda, cfg, engine="auto"):
    x, router = wl.make_activations(cfg, 0)
    w = wl.make_weights(cfg, wl.layer_seed(0))
    lw = dev.LayerWeights(w, cfg.E)
    got, inter = _layer_gpu(torch_cuda, cfg, x, router, lw, engine=engine)
    del lw
    _check_layer_integer_stages(cfg, x, router, inter)
    ref = oracle.moe_layer(x, router, w, cfg.k)
    check_tol(bf16f(got), ref["out"], f"layer {cfg.name} [{engine}] out")


FULL_LAYER = ["tiny", "decode1", "decode4", "prefill512", "zipf8192", "uniform8192",
              "tiny_affine", "prefill512_affine", "zipf8192_affine"]


@pytest.mark.parametrize("name", FULL_LAYER)
def test_layer_forward_parity_full(torch_cuda, name):
    """Every output element against the oracle, including both 8192-token layers (the wide
    engine's default regime) and the per-group affine bias recipe."""
    cfg = wl.CONFIGS[name]
    say(f"layer {name}: full oracle")
    _layer_full_check(torch_cuda, cfg)


@pytest.mark.parametrize("routing", ["natural", "zipf"])
def test_layer_forward_paired_multi_tile_groups(torch_cuda, routing):
    """1000 tokens (about 31 rows per expert on average, still the resident engine): the
    paired gate_up/down launch with groups of more than 32 rows (two or more tiles each, so
    a tile's down work waits on gate_up chunks of several workgroups), with natural and
    Zipf-skewed routing (empty groups, one group of hundreds of rows), every element."""
    cfg = wl.MoEConfig(f"paired1000_{routing}", 1000, 2048, 256, 8, 512, routing=routing)
    plan = L.moe_layer_plan(L.shape(cfg.T, cfg.D, cfg.E, cfg.k, cfg.F))
    assert plan.gemm_engine == L.MOE_ENGINE_RESIDENT and plan.paired == 1
    say(f"layer {cfg.name}: full oracle (paired launch)")
    _layer_full_check(torch_cuda, cfg)


@pytest.mark.parametrize("engine", ENGINES)
@pytest.mark.parametrize("name", ["tiny", "prefill512"])
def test_layer_forward_parity_engines(torch_cuda, name, engine):
    """The same layers through each engine, also those the automatic choice does not pick."""
    cfg = wl.CONFIGS[name]
    say(f"layer {name} [{engine}]: full oracle")
    _layer_full_check(torch_cuda, cfg, engine)


def test_layer_forward_long_sampled(torch_cuda):
    """The 32768-token chunk: integer stages on every token, outputs on 4096 seeded tokens
    (first and last included) per layer for each of the four distinct weight sets, run back
    to back on the same x."""
    cfg = wl.CONFIGS["long32768"]
    x, router = wl.make_activations(cfg, 0)
    rng = np.random.default_rng(2024)
    toks = np.unique(np.concatenate([[0, cfg.T - 1], rng.choice(cfg.T, 4094, replace=False)]))
    assert len(toks) >= 4096
    for layer in range(cfg.n_layers):
        say(f"layer long32768 #{layer}: {len(toks)} sampled tokens")
        w = wl.make_weights(cfg, wl.layer_seed(layer))
        lw = dev.LayerWeights(w, cfg.E)
        got, inter = _layer_gpu(torch_cuda, cfg, x, router, lw)
        del lw
        _check_layer_integer_stages(cfg, x, router, inter)
        ref, _, _ = oracle.moe_out_for_tokens(x, router, w, cfg.k, toks)
        check_tol(bf16f(got[toks]), ref, f"layer long32768 #{layer} sampled out")


def test_layer_forward_chunked(torch_cuda):
    """moe_layer_forward_chunked over 5000 tokens in chunks of 2048 (two chunks on the router's
    bf16 planes, the second reusing them, and a last chunk of 904 on the fp32-from-R router),
    every element against the oracle, and its workspace that of one chunk."""
    torch = torch_cuda
    cfg = wl.MoEConfig("chunked", 5000, 1024, 64, 4, 256)
    x, router = wl.make_activations(cfg, 3)
    w = wl.make_weights(cfg, 55)
    lw = dev.LayerWeights(w, cfg.E)
    shp = L.shape(cfg.T, cfg.D, cfg.E, cfg.k, cfg.F)
    chunk = 2048
    nb = L.moe_chunked_workspace_bytes(shp, chunk)
    assert nb == L.moe_workspace_bytes(L.shape(chunk, cfg.D, cfg.E, cfg.k, cfg.F))
    assert nb < L.moe_workspace_bytes(shp)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    out = torch.empty((cfg.T, cfg.D), dtype=torch.int16, device="cuda")
    xd, rd = dev.to_device(x), dev.to_device(router)
    L.moe_layer_forward_chunked(shp, xd, rd, lw.experts, lw.shared, out, chunk, ws)
    torch.cuda.synchronize()
    ref = oracle.moe_layer(x, router, w, cfg.k)
    check_tol(bf16f(dev.to_host(out, np.uint16)), ref["out"], "chunked layer")


def test_layer_forward_chunked_long(torch_cuda):
    """The 32768-token layer in four chunks of 8192 with a workspace of one chunk: outputs on
    4096 seeded tokens against the oracle, and every output within the tolerance of the
    single-call layer's (both on the wide engine)."""
    torch = torch_cuda
    cfg = wl.CONFIGS["long32768"]
    x, router = wl.make_activations(cfg, 0)
    w = wl.make_weights(cfg, wl.layer_seed(1))
    lw = dev.LayerWeights(w, cfg.E)
    shp = L.shape(cfg.T, cfg.D, cfg.E, cfg.k, cfg.F)
    xd, rd = dev.to_device(x), dev.to_device(router)
    whole = torch.empty((cfg.T, cfg.D), dtype=torch.int16, device="cuda")
    ws = dev.workspace(shp)
    L.moe_layer_forward(shp, xd, rd, lw.experts, lw.shared, whole, ws)
    torch.cuda.synchronize()
    del ws
    nb = L.moe_chunked_workspace_bytes(shp, 8192)
    say(f"chunked long32768: workspace {nb / 2**20:.0f} MiB against "
        f"{L.moe_workspace_bytes(shp) / 2**20:.0f} MiB in one call")
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    part = torch.empty_like(whole)
    L.moe_layer_forward_chunked(shp, xd, rd, lw.experts, lw.shared, part, 8192, ws)
    torch.cuda.synchronize()
    got = dev.to_host(part, np.uint16)
    rng = np.random.default_rng(2025)
    toks = np.unique(np.concatenate([[0, 8191, 8192, cfg.T - 1],
                                     rng.choice(cfg.T, 4092, replace=False)]))
    ref, _, _ = oracle.moe_out_for_tokens(x, router, w, cfg.k, toks)
    check_tol(bf16f(got[toks]), ref, "chunked long32768 sampled out")
    a, b = bf16f(got), bf16f(dev.to_host(whole, np.uint16))
    rms = math.sqrt(float(np.mean(b * b)))
    assert np.all(np.abs(a - b) <= ATOL_RMS * rms + RTOL * np.abs(b))


def test_layer_forward_no_shared(torch_cuda):
    cfg = wl.CONFIGS["tiny"]
    x, router = wl.make_activations(cfg, 0)
    w = wl.make_weights(cfg, 1000)
    lw = dev.LayerWeights(w, cfg.E)
    got, inter = _layer_gpu(torch_cuda, cfg, x, router, lw, with_shared=False)
    _check_layer_integer_stages(cfg, x, router, inter, with_shared=False)
    ref = oracle.moe_layer(x, router, w, cfg.k, with_shared=False)
    check_tol(bf16f(got), ref["out"], "tiny without shared expert")


@pytest.mark.parametrize("engine", ENGINES)
@pytest.mark.parametrize("shape", [(33, 128, 40, 32, 64), (40, 64, 1000, 4, 64), (300, 192, 8, 1, 192),
                                   (1500, 320, 4, 2, 192), (1500, 256, 4, 2, 128),
                                   (77, 384, 24, 3, 256), (5, 128, 16, 4, 128),
                                   (300, 512, 24, 3, 256), (40, 1024, 64, 4, 512),
                                   (64, 64, 1024, 16, 64), (1100, 256, 64, 8, 128)])
def test_layer_forward_odd_shapes(torch_cuda, shape, engine):
    """Wide top-k (k = 32), many experts (E = 1000, and E = 1024, the most the interface takes,
    with 613 of them touched), K % 128 == 64 (D = F = 192), a single expert per token, and
    T * k > 8192 with T > 1024 (the chunked histogram, scan and scatter with the tile map
    written by the scan launch), every output element checked."""
    T, D, E, k, F = shape
    cfg = wl.MoEConfig("odd", T, D, E, k, F, bias="affine")
    x, router = wl.make_activations(cfg, 5)
    w = wl.make_weights(cfg, 77)
    lw = dev.LayerWeights(w, cfg.E)
    got, inter = _layer_gpu(torch_cuda, cfg, x, router, lw, engine=engine)
    _check_layer_integer_stages(cfg, x, router, inter)
    ref = oracle.moe_layer(x, router, w, cfg.k)
    check_tol(bf16f(got), ref["out"], f"layer {shape} [{engine}]")


def test_layer_forward_deterministic(torch_cuda):
    cfg = wl.CONFIGS["prefill512"]
    x, router = wl.make_activations(cfg, 0)
    lw = dev.LayerWeights(wl.make_weights(cfg, 1000), cfg.E)
    a, _ = _layer_gpu(torch_cuda, cfg, x, router, lw)
    b, _ = _layer_gpu(torch_cuda, cfg, x, router, lw)
    assert np.array_equal(a, b)


def test_layer_stage_events(torch_cuda):
    """moe_layer_forward_ex with stage events records all six and gives the same output."""
    torch = torch_cuda
    cfg = wl.CONFIGS["tiny"]
    x, router = wl.make_activations(cfg, 0)
    lw = dev.LayerWeights(wl.make_weights(cfg, 1000), cfg.E)
    plain, _ = _layer_gpu(torch, cfg, x, router, lw)
    shp = L.shape(cfg.T, cfg.D, cfg.E, cfg.k, cfg.F)
    ws = dev.workspace(shp)
    out = torch.empty((cfg.T, cfg.D), dtype=torch.int16, device="cuda")
    evs = [dev.hip_event() for _ in range(L.N_STAGE_EVENTS)]
    L.moe_layer_forward_ex(shp, dev.to_device(x), dev.to_device(router), lw.experts, lw.shared,
                           out, ws, L.layer_opts("auto", evs))
    torch.cuda.synchronize()
    assert all(dev.hip_elapsed_ms(evs[i], evs[i + 1]) >= 0 for i in range(L.N_STAGE_EVENTS - 1))
    for e in evs:
        dev.hip_event_destroy(e)
    assert np.array_equal(dev.to_host(out, np.uint16), plain)


@pytest.mark.parametrize("shape", [(2100, 512, 200, 6, 256), (3000, 256, 17, 3, 128)])
def test_layer_many_tokens_off_shapes(torch_cuda, shape):
    """Many-token layers away from the Qwen-like shape, every element against the oracle and
    the routing outputs on every token: 200 experts (a partial 128-expert router tile),
    12,600 pairs (count / scan / scatter), about 63 rows per group (128-row tiles); and 17
    experts of about 530 rows with d_ff 128 (a down K below one 256-wide stage)."""
    T, D, E, k, F = shape
    cfg = wl.MoEConfig("many_off", T, D, E, k, F)
    x, router = wl.make_activations(cfg, 21)
    w = wl.make_weights(cfg, 77)
    lw = dev.LayerWeights(w, cfg.E)
    say(f"many-token layer {shape}")
    got, inter = _layer_gpu(torch_cuda, cfg, x, router, lw)
    _check_layer_integer_stages(cfg, x, router, inter)
    ref = oracle.moe_layer(x, router, w, cfg.k)
    check_tol(bf16f(got), ref["out"], f"many-token layer {shape}")


# ----------------------------------------------------------------------------- decode sizes
DECODE_SHAPES = [(1, 2048, 256, 8, 512), (4, 2048, 256, 8, 512), (16, 2048, 256, 8, 512),
                 (4, 256, 1000, 32, 128), (3, 512, 40, 8, 64), (16, 256, 16, 2, 128)]


@pytest.mark.parametrize("engine", ["decode", "resident"])
@pytest.mark.parametrize("shape", DECODE_SHAPES)
def test_layer_decode_sizes(torch_cuda, shape, engine):
    """T <= 16: the decode-sized chain (plan, gate_up per slot and slice, down fused with the
    combine) and the grouped chain on the same layers, every element against the oracle and
    the routing outputs (ordered top-k, offsets, permuted rows) on every token.  Shapes: the
    Qwen-like layer at 1, 4 and 16 tokens (16 x 8 = 128 pairs, the most the chain takes),
    k = 32 with 1000 experts (128 pairs, E > 256), F = 64 (one 64-wide group per down row)."""
    T, D, E, k, F = shape
    cfg = wl.MoEConfig("dec", T, D, E, k, F)
    x, router = wl.make_activations(cfg, 11)
    w = wl.make_weights(cfg, 99)
    lw = dev.LayerWeights(w, cfg.E)
    say(f"decode-sized layer {shape} [{engine}]")
    got, inter = _layer_gpu(torch_cuda, cfg, x, router, lw, engine=engine)
    _check_layer_integer_stages(cfg, x, router, inter)
    ref = oracle.moe_layer(x, router, w, cfg.k)
    check_tol(bf16f(got), ref["out"], f"decode-sized layer {shape} [{engine}]")


def test_layer_decode_no_shared(torch_cuda):
    cfg = wl.MoEConfig("dec_ns", 4, 2048, 256, 8, 512)
    x, router = wl.make_activations(cfg, 12)
    w = wl.make_weights(cfg, 98)
    lw = dev.LayerWeights(w, cfg.E)
    got, inter = _layer_gpu(torch_cuda, cfg, x, router, lw, with_shared=False, engine="decode")
    _check_layer_integer_stages(cfg, x, router, inter, with_shared=False)
    ref = oracle.moe_layer(x, router, w, cfg.k, with_shared=False)
    check_tol(bf16f(got), ref["out"], "decode-sized layer without the shared expert")


def test_decode_engine_rejects_large_batches(torch_cuda):
    cfg = wl.MoEConfig("dec_big", 17, 2048, 256, 8, 512)
    shp = L.shape(cfg.T, cfg.D, cfg.E, cfg.k, cfg.F)
    x, router = wl.make_activations(cfg, 0)
    lw = dev.LayerWeights(wl.make_weights(cfg, 1000), cfg.E)
    out = torch_cuda.empty((cfg.T, cfg.D), dtype=torch_cuda.int16, device="cuda")
    with pytest.raises(L.MoEError) as ei:
        L.moe_layer_forward_ex(shp, dev.to_device(x), dev.to_device(router), lw.experts,
                               lw.shared, out, dev.workspace(shp), L.layer_opts("decode"))
    assert ei.value.status == L.MOE_ERR_SHAPE


@pytest.mark.parametrize("name", ["decode1", "decode4"])
def test_layer_decode_graph_replay(torch_cuda, name):
    """The decode-sized layer captured into a HIP graph (torch.cuda.CUDAGraph) and replayed
    five times with new inputs copied in and eager work between replays: every replay equals
    the eager call on the same inputs, bit for bit."""
    torch = torch_cuda
    cfg = wl.CONFIGS[name]
    lw = dev.LayerWeights(wl.make_weights(cfg, wl.layer_seed(0)), cfg.E)
    shp = L.shape(cfg.T, cfg.D, cfg.E, cfg.k, cfg.F)
    ws = dev.workspace(shp)
    xs, rs = [], []
    for seed in range(5):
        x, r = wl.make_activations(cfg, seed)
        xs.append(dev.to_device(x))
        rs.append(dev.to_device(r))
    xin, rin = torch.empty_like(xs[0]), torch.empty_like(rs[0])
    out = torch.empty((cfg.T, cfg.D), dtype=torch.int16, device="cuda")
    # eager references
    refs = []
    for i in range(5):
        o = torch.empty_like(out)
        L.moe_layer_forward(shp, xs[i], rs[i], lw.experts, lw.shared, o, ws)
        refs.append(o)
    torch.cuda.synchronize()
    xin.copy_(xs[0])
    rin.copy_(rs[0])
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # one warm call on the side stream before capture
        L.moe_layer_forward(shp, xin, rin, lw.experts, lw.shared, out, ws, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        L.moe_layer_forward(shp, xin, rin, lw.experts, lw.shared, out, ws)
    for i in range(5):
        xin.copy_(xs[i])
        rin.copy_(rs[i])
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, refs[i]), f"replay {i} differs from the eager call"
        junk = torch.randn(1 << 16, device="cuda").sum()  # eager work between replays
        torch.cuda.synchronize()
        del junk
