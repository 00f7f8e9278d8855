#!/usr/bin/env python3
"""MoE-layer throughput on one MI355X.

A step is one moe_layer_forward (routing, histogram/scan/scatter, grouped gate_up +
SwiGLU and grouped down (one launch at 512 tokens), weighted combine) over one batch of synthetic tokens whose inputs
are resident in HBM.  The headline workload is the 512-token prefill of a
Qwen3.6-35B-A3B-shaped layer (d_model 2048, 256 experts top-8 + 1 shared expert, d_ff 512,
int4 weights with bf16 scale and bias per 64); the 8192-token prefill with Zipf-skewed
routing is measured in the same run and reported in the same line (`zipf8192`), and so is the
per-layer latency of the decode-sized layer at 1 and 4 tokens, eager and as graph replays
(`decode`), and the 32768-token layer as one call and in bounded chunks (`long32768`).  Four
distinct weight sets (455 MB each; together more than the 256 MB Infinity Cache) rotate so
that every step streams its weights from HBM.

Prints one JSON line: value = tokens/s at T=512, the roofline of the dominant kernel
(the launch that runs grouped gate_up + SwiGLU and down at 512 tokens, the grouped gate_up
at 8192; timed inside the timed region with two HIP events that the library records on the
layer's stream around it, on every fourth timed step; the events are created without the
system-scope fence of a default event) and of the whole layer, the same for the 8192-token
layer, a measured HBM ceiling (a plain device copy and a streaming read, timed with events)
and the CPU oracle's rate on a bounded sample.  The per-stage breakdown (stage_us) comes
from a separate pass after each timed region with an event at every stage boundary, since
those events themselves cost a few microseconds per step; the per-call latency
distribution (latency: p10 / p50 / p90) from another pass with one event before and one
after each call.  `staged_ablation` times the same layer through the staged entry points,
with the group offsets kept on the device and with the host reading them back.

    python bench.py [--steps K] [--warmup W] [--config prefill512|zipf8192|uniform8192|...]
                    [--no-secondary] [--no-decode] [--no-long] [--no-attention]
                    [--no-cpu-baseline] [--copy-probe]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, AMD published
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 MFMA, AMD published
RIDGE = BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
METRIC = "MoE-layer tokens/sec at T=512 and T=8192; % of HBM / MFMA roofline"
SECONDARY = "zipf8192"          # the T=8192 half of the metric, measured in the same run
EV_EVERY = 4                    # timed steps per pair of events around the dominant launch
N_LAT = 100                     # calls in the per-call latency pass (p10 / p50 / p90)

# the dominant kernel for each workload: the grouped gate_up (wide-tile engine), or, where
# the library runs gate_up and down as one launch (moe_layer_plan: paired), that launch
KERNEL_LABEL = {
    "wide": "grouped gate_up + SwiGLU (q4_wide_kernel<true, 1>)",
    "resident": "grouped gate_up + SwiGLU (q4_resident_kernel<true, 4>)",
    "paired": "grouped gate_up + SwiGLU then down, one launch (q4_resident_pair_kernel<4, 2>)",
}

# FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the dominant kernel and of the plain 1 GiB
# copy kernel of --copy-probe, read in the same rocprofv3 --pmc runs; the build they were
# taken on is named in the matching profiles/ summary.  A workload missing here reports
# traffic null.
TRAFFIC = {
    # commit b94ebe5 (profiles/grouped_gemms_pair_prefill512_traffic.md)
    "prefill512": {"fetch_kib": 248694.3, "write_kib": 27782.2,
                   "copy_fetch_kib": 524300.0, "copy_write_kib": 1048576.0,
                   "copy_bytes": 1 << 30},
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # the first ~100 layer calls of a process run a few percent slower (measured: 166 against
    # 160 us per layer at 512 tokens right after 50 warm-up calls), so the default warm-up
    # is longer than that
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--config", default="prefill512")
    ap.add_argument("--weight-sets", type=int, default=4)
    ap.add_argument("--no-attention", action="store_true",
                    help="skip the grouped-query decode attention object")
    ap.add_argument("--no-long", action="store_true",
                    help="skip the 32768-token layer (single call vs bounded chunks)")
    ap.add_argument("--no-decode", action="store_true",
                    help="skip the decode-sized latency object (T=1 and T=4)")
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the 8192-token Zipf layer measured after the headline one")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run one plain 1 GiB device copy (for scaling PMC byte counters)")
    ap.add_argument("--sweep", action="store_true",
                    help="instead of the layer: the grouped gate_up GEMM alone with n_e rows in "
                         "each of the 257 groups, n_e = 1 .. 2048, per engine (regime evidence)")
    ap.add_argument("--sweep-sizes", default="1,2,4,8,16,32,64,128,256,512,1024,2048")
    ap.add_argument("--sweep-engines", default="resident,wide")
    return ap.parse_args()


def gate_up_algorithmic(cfg, touched_groups):
    """Bytes and flops the grouped gate_up must move/do at minimum: touched groups' codes +
    scale + bias (2F x D weights at 0.5625 B each), x read once, activations written."""
    wbytes = touched_groups * 2 * cfg.F * cfg.D * (4 + 32 / 64) / 8
    bytes_ = wbytes + cfg.T * cfg.D * 2 + (cfg.k + 1) * cfg.T * cfg.F * 2
    flops = 2.0 * (cfg.k + 1) * cfg.T * 2 * cfg.F * cfg.D
    return bytes_, flops


def pair_algorithmic(cfg, touched_groups):
    """Bytes and flops of gate_up + SwiGLU and down in one launch: the touched groups'
    codes + scale + bias (3 F x D weights at 0.5625 B each), x read once, the activations
    written and read back, y written."""
    rows = (cfg.k + 1) * cfg.T
    wbytes = touched_groups * 3 * cfg.F * cfg.D * (4 + 32 / 64) / 8
    bytes_ = wbytes + cfg.T * cfg.D * 2 + 2 * rows * cfg.F * 2 + rows * cfg.D * 2
    flops = 2.0 * rows * 3 * cfg.F * cfg.D
    return bytes_, flops


def roofline(bytes_, flops, seconds):
    """The bound (HBM below the ridge, bf16 MFMA above) and the achieved fraction of it."""
    if flops / bytes_ < RIDGE:
        r = {"bound": "hbm", "achieved": bytes_ / seconds / 1e9, "peak": HBM_PEAK_GBS,
             "unit": "GB/s"}
    else:
        r = {"bound": "mfma", "achieved": flops / seconds / 1e12, "peak": BF16_PEAK_TFLOPS,
             "unit": "TFLOP/s"}
    r["frac"] = r["achieved"] / r["peak"]
    return r


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg, x, router, w):
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max((i.get("num_threads", 1) for i in threadpool_info()
                     if i.get("user_api") == "blas"), default=1)
    except Exception:  # noqa: BLE001
        cores = os.cpu_count() or 1
    if cfg.T <= 512:
        # the whole layer, repeated until about 10 s of CPU work (at most 8 times)
        reps, t0 = 0, time.perf_counter()
        while reps < 8 and (reps == 0 or time.perf_counter() - t0 < 10.0):
            oracle.moe_layer(x, router, w, cfg.k)
            reps += 1
        dt = time.perf_counter() - t0
        n = cfg.T * reps
        sample = f"the whole {cfg.T}-token layer (routing, all experts, combine), fp64, {reps} times"
    else:
        toks = np.random.default_rng(7).integers(0, cfg.T, 128)
        t0 = time.perf_counter()
        oracle.moe_out_for_tokens(x, router, w, cfg.k, toks)
        dt = time.perf_counter() - t0
        n, sample = len(toks), f"128 sampled tokens of the {cfg.T}-token layer, fp64"
    return {"value": n / dt, "unit": "tokens/s", "cores": int(cores), "cpu_model": cpu_model(),
            "kind": "oracle", "sample": sample, "seconds": round(dt, 3)}


def measure(cfg, sets, steps, warmup, torch, L, dev, wl):
    """Time `steps` layer calls of `cfg` (after `warmup` untimed ones) with the gate_up events
    inside; then a breakdown pass with every stage event.  Returns the figures and the group
    offsets of the last call."""
    x, router = wl.make_activations(cfg, 0)
    xd, rd = dev.to_device(x), dev.to_device(router)
    shp = L.shape(cfg.T, cfg.D, cfg.E, cfg.k, cfg.F)
    ws = dev.workspace(shp)
    out = torch.empty((cfg.T, cfg.D), dtype=torch.int16, device="cuda")
    stream = torch.cuda.current_stream()
    nst = L.N_STAGE_EVENTS
    GU = 2  # events[2]: after the permutation, events[3]: after gate_up (or after both
    #         GEMMs when they run as one launch)
    plan = L.moe_layer_plan(shp)
    paired = bool(plan.paired)
    eng = {L.MOE_ENGINE_WIDE: "wide", L.MOE_ENGINE_RESIDENT: "resident"}.get(plan.gemm_engine)
    n_brk = min(steps, 20)
    # events exist only while their pass runs (each pass creates and destroys its own): the
    # timed steps that record the two events around the dominant launch
    sampled = [i for i in range(steps) if i % EV_EVERY == 0]
    evs = {i: (dev.hip_event(), dev.hip_event()) for i in sampled}
    opts_gu = {i: L.layer_opts("auto", [a if j == GU else b if j == GU + 1 else None for j in range(nst)])
               for i, (a, b) in evs.items()}

    def step(i, opts=None):
        lw = sets[i % len(sets)]
        if opts is None:
            L.moe_layer_forward(shp, xd, rd, lw.experts, lw.shared, out, ws, stream=stream)
        else:
            L.moe_layer_forward_ex(shp, xd, rd, lw.experts, lw.shared, out, ws, opts, stream=stream)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    log(f"bench: {cfg.name}: warmup done ({warmup} steps)")

    # ---- timed region: exactly K steps; every EV_EVERY-th step (the first included) records
    # the two events around the dominant launch (an event costs about a microsecond of
    # stream time, so the others run without)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i, opts_gu.get(i))
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / steps
    gu_ms = float(np.mean([dev.hip_elapsed_ms(a, b) for a, b in evs.values()]))
    for a, b in evs.values():
        dev.hip_event_destroy(a)
        dev.hip_event_destroy(b)
    log(f"bench: {cfg.name}: {steps} steps in {elapsed * 1e3:.2f} ms ({ms_per_step:.4f} ms/step), "
        f"{'gate_up + down (one launch)' if paired else 'gate_up'} {gu_ms * 1e3:.1f} us")

    # ---- per-call latency distribution (reporting only), right after the timed region:
    # N_LAT calls, each between one event before its first kernel and one after its last
    # (an event's own cost, one to two microseconds of stream time, is inside every figure)
    lat = [[dev.hip_event() for _ in range(2)] for _ in range(N_LAT)]
    opts_lat = [L.layer_opts("auto", [a] + [None] * (nst - 2) + [b]) for a, b in lat]
    for i in range(N_LAT):
        step(i, opts_lat[i])
    torch.cuda.synchronize()
    lat_us = np.array([dev.hip_elapsed_ms(a, b) * 1e3 for a, b in lat])
    p10, p50, p90 = (float(v) for v in np.percentile(lat_us, [10, 50, 90]))
    latency = {"calls": N_LAT, "p10_us": p10, "p50_us": p50, "p90_us": p90,
               "tokens_per_s_at_p50": cfg.T / (p50 * 1e-6)}
    log(f"bench: {cfg.name}: per-call latency over {N_LAT} calls: p10 {p10:.1f} us, p50 {p50:.1f} us, "
        f"p90 {p90:.1f} us")
    for a, b in lat:
        dev.hip_event_destroy(a)
        dev.hip_event_destroy(b)

    # ---- per-stage breakdown (reporting only, outside the timed region)
    brk = [[dev.hip_event() for _ in range(nst)] for _ in range(n_brk)]
    opts_all = [L.layer_opts("auto", row) for row in brk]
    for i in range(n_brk):
        step(i, opts_all[i])
    torch.cuda.synchronize()
    names = ["route", "permute", "gate_up", "down", "combine"]
    if paired:  # events [3] and [4] both follow the one GEMM launch
        names = ["route", "permute", "gate_up_and_down", None, "combine"]
    stage_ms = {n: float(np.mean([dev.hip_elapsed_ms(brk[i][j], brk[i][j + 1]) for i in range(n_brk)]))
                for j, n in enumerate(names) if n}
    log(f"bench: {cfg.name}: breakdown (events at every stage): "
        + ", ".join(f"{k}={v * 1e3:.1f}us" for k, v in stage_ms.items()))

    for row in brk:
        for e in row:
            dev.hip_event_destroy(e)

    lay = L.moe_workspace_layout(shp)
    offs = ws[lay.offsets:lay.offsets + 4 * (cfg.E + 2)].cpu().numpy().view(np.int32)
    touched = int(np.count_nonzero(np.diff(offs[:cfg.E + 1]))) + 1  # + the shared expert
    counts = np.diff(offs[:cfg.E + 1])
    gb, gf = (pair_algorithmic if paired else gate_up_algorithmic)(cfg, touched)
    roof = roofline(gb, gf, gu_ms * 1e-3)
    t = TRAFFIC.get(cfg.name)
    if t:
        scale_f = t["copy_bytes"] / (t["copy_fetch_kib"] * 1024)
        scale_w = t["copy_bytes"] / (t["copy_write_kib"] * 1024)
        roof["traffic"] = t["fetch_kib"] * 1024 * scale_f + t["write_kib"] * 1024 * scale_w
    else:
        roof["traffic"] = None
    roof["kernel"] = KERNEL_LABEL["paired" if paired else eng] if (paired or eng) else "grouped gate_up"
    roof["algorithmic_bytes"] = gb
    roof["algorithmic_flops"] = gf
    roof["kernel_us"] = gu_ms * 1e3
    roof["kernel_timed_steps"] = len(sampled)
    layer = roofline(float(wl.algorithmic_bytes(cfg, touched)), float(wl.expert_flops(cfg)),
                     ms_per_step * 1e-3)
    layer["algorithmic_bytes"] = float(wl.algorithmic_bytes(cfg, touched))
    layer["algorithmic_flops"] = float(wl.expert_flops(cfg))
    return {
        "ms_per_step": ms_per_step, "value": cfg.T / (ms_per_step * 1e-3),
        "stage_us": {k: v * 1e3 for k, v in stage_ms.items()},
        "latency": latency,
        "touched_groups": touched,
        "rows_per_group": {"min": int(counts.min()), "median": float(np.median(counts)),
                           "max": int(counts.max()), "empty": int((counts == 0).sum())},
        "roofline": roof, "layer_roofline": layer,
    }, (x, router)


def measure_staged(cfg, sets, torch, L, dev, wl, calls=40):
    """The layer through the staged entry points (moe_route, moe_permute, four
    moe_grouped_gemm_q4 calls: routed gate_up + SwiGLU, routed down, shared gate_up + SwiGLU,
    shared down; moe_combine), every one on the stream with the group offsets on the device,
    and the same chain with the host reading the offsets back between the permutation and
    the GEMMs (a device-to-host copy and a stream synchronisation, as a host-sized launch
    would need): the analogue of the pages' host-synchronisation ablation.  Per-layer times
    are wall-clock over `calls` layers bracketed by synchronisations, rotating the weight
    sets."""
    T, D, E, k, F = cfg.T, cfg.D, cfg.E, cfg.k, cfg.F
    x, router = wl.make_activations(cfg, 0)
    xd, rd = dev.to_device(x), dev.to_device(router)
    shp = L.shape(T, D, E, k, F)
    ws = dev.workspace(shp)
    i32, i16 = torch.int32, torch.int16
    idx = torch.empty((T, k), dtype=i32, device="cuda")
    wts = torch.empty((T, k), dtype=torch.float32, device="cuda")
    off = torch.empty(E + 1, dtype=i32, device="cuda")
    st = torch.empty(T * k, dtype=i32, device="cuda")
    sr = torch.empty(T * k, dtype=i32, device="cuda")
    off_sh = torch.tensor([0, T], dtype=i32, device="cuda")
    act = torch.empty((T * k, F), dtype=i16, device="cuda")
    y = torch.empty((T * k, D), dtype=i16, device="cuda")
    s_act = torch.empty((T, F), dtype=i16, device="cuda")
    S = torch.empty((T, D), dtype=i16, device="cuda")
    out = torch.empty((T, D), dtype=i16, device="cuda")
    gws_n = max(L.moe_grouped_gemm_q4_workspace_bytes(E, T * k, T, D),
                L.moe_grouped_gemm_q4_workspace_bytes(E, T * k, T * k, F),
                L.moe_grouped_gemm_q4_workspace_bytes(1, T, T, D),
                L.moe_grouped_gemm_q4_workspace_bytes(1, T, T, F))
    gws = torch.empty(max(gws_n, 256), dtype=torch.uint8, device="cuda")

    def layer(i, host_sync):
        lw = sets[i % len(sets)]
        ex, sh = lw.experts, lw.shared
        L.moe_route(shp, xd, rd, idx, wts, ws)
        L.moe_permute(shp, idx, off, st, sr, ws)
        if host_sync:
            off.cpu()  # device-to-host copy: the host waits for the stream
        L.moe_grouped_gemm_q4(E, T * k, 2 * F, D, xd, T, st, off, ex.gate_up, 1, act, gws)
        L.moe_grouped_gemm_q4(E, T * k, D, F, act, T * k, None, off, ex.down, 0, y, gws)
        L.moe_grouped_gemm_q4(1, T, 2 * F, D, xd, T, None, off_sh, sh.gate_up, 1, s_act, gws)
        L.moe_grouped_gemm_q4(1, T, D, F, s_act, T, None, off_sh, sh.down, 0, S, gws)
        L.moe_combine(shp, y, sr, wts, S, out)

    res = {}
    for name, hs in (("device_offsets", False), ("host_sync", True)):
        for i in range(8):
            layer(i, hs)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(calls):
            layer(i, hs)
        torch.cuda.synchronize()
        res[name + "_us_per_layer"] = (time.perf_counter() - t0) / calls * 1e6
    log(f"bench: {cfg.name}: staged entry points {res['device_offsets_us_per_layer']:.1f} us per layer, "
        f"with the host reading the offsets {res['host_sync_us_per_layer']:.1f} us")
    return res


def measure_decode(cfg, sets, torch, L, dev, wl, layers=200):
    """Per-layer latency of the decode-sized layer (T <= 16): `layers` back-to-back layer calls
    rotating the weight sets, issued eagerly and as replays of one captured graph of four
    layers (one per weight set, so each layer's weights come from HBM).  The HBM floor is the
    layer's algorithmic bytes (touched experts' codes, scales and biases, the router, x and
    out) at the published 8 TB/s."""
    x, router = wl.make_activations(cfg, 0)
    xd, rd = dev.to_device(x), dev.to_device(router)
    shp = L.shape(cfg.T, cfg.D, cfg.E, cfg.k, cfg.F)
    ws = dev.workspace(shp)
    out = torch.empty((cfg.T, cfg.D), dtype=torch.int16, device="cuda")
    n = len(sets)

    def layer(i, stream):
        lw = sets[i % n]
        L.moe_layer_forward(shp, xd, rd, lw.experts, lw.shared, out, ws, stream=stream)

    cur = torch.cuda.current_stream()
    for i in range(2 * n):
        layer(i, cur)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(layers):
        layer(i, cur)
    torch.cuda.synchronize()
    eager_us = (time.perf_counter() - t0) * 1e6 / layers

    side = torch.cuda.Stream()
    side.wait_stream(cur)
    with torch.cuda.stream(side):
        for i in range(n):
            layer(i, side)
    cur.wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cap = torch.cuda.current_stream()
        for i in range(n):
            layer(i, cap)
    for _ in range(4):
        g.replay()
    torch.cuda.synchronize()
    reps = max(1, layers // n)
    t0 = time.perf_counter()
    for _ in range(reps):
        g.replay()
    torch.cuda.synchronize()
    graph_us = (time.perf_counter() - t0) * 1e6 / (reps * n)
    del g

    lay = L.moe_workspace_layout(shp)
    offs = ws[lay.offsets:lay.offsets + 4 * (cfg.E + 2)].cpu().numpy().view(np.int32)
    touched = int(np.count_nonzero(np.diff(offs[:cfg.E + 1]))) + 1
    nbytes = float(wl.algorithmic_bytes(cfg, touched))
    floor_us = nbytes / (HBM_PEAK_GBS * 1e9) * 1e6
    log(f"bench: {cfg.name}: eager {eager_us:.1f} us/layer, graph replay {graph_us:.1f} us/layer, "
        f"HBM floor {floor_us:.2f} us ({touched} experts touched)")
    return {"T": cfg.T, "touched_groups": touched, "eager_us_per_layer": eager_us,
            "graph_us_per_layer": graph_us, "algorithmic_bytes": nbytes,
            "hbm_floor_us": floor_us, "floor_frac_graph": floor_us / graph_us,
            "layers_timed": layers}


def measure_long(cfg, sets, torch, L, dev, wl, chunks=(8192, 16384), reps=3):
    """The long-prompt layer (T = 32768) as one call and as moe_layer_forward_chunked in chunks
    of each size in `chunks` tokens with a workspace of one chunk: per-layer time over `reps`
    passes of the four weight sets, and the workspace sizes."""
    x, router = wl.make_activations(cfg, 0)
    xd, rd = dev.to_device(x), dev.to_device(router)
    shp = L.shape(cfg.T, cfg.D, cfg.E, cfg.k, cfg.F)
    out = torch.empty((cfg.T, cfg.D), dtype=torch.int16, device="cuda")
    res = {"T": cfg.T}
    for mode in ["single"] + [f"chunked_{c}" for c in chunks]:
        if mode == "single":
            nb = L.moe_workspace_bytes(shp)
            ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
            call = lambda lw: L.moe_layer_forward(shp, xd, rd, lw.experts, lw.shared, out, ws)
        else:
            chunk = int(mode.split("_")[1])
            nb = L.moe_chunked_workspace_bytes(shp, chunk)
            ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
            call = lambda lw, chunk=chunk, ws=ws: L.moe_layer_forward_chunked(
                shp, xd, rd, lw.experts, lw.shared, out, chunk, ws)
        for lw in sets:
            call(lw)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            for lw in sets:
                call(lw)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / (reps * len(sets))
        res[mode] = {"ms_per_layer": ms, "tokens_per_s": cfg.T / (ms * 1e-3), "workspace_bytes": nb}
        log(f"bench: {cfg.name} {mode}: {ms:.3f} ms/layer, workspace {nb / 1e6:.1f} MB")
        del ws
    return res


def measure_attention(torch, L, dev, wl, reps=200):
    """Grouped-query decode attention (one query token, 16 query heads on two KV heads, head
    dim 128) at 4K, 32K and 128K cached positions: time per call (the two kernels, partial and
    reduce) as replays of a captured graph of eight calls (and, for reference, over `reps`
    calls issued one by one), and the cache bytes read per second."""
    res = {}
    for name in ("attn4k", "attn32k", "attn128k"):
        n_q, n_kv, d, ctx = wl.ATTN_CONFIGS[name]
        q, k, v = wl.make_attention_inputs(n_q, n_kv, d, ctx, seed=0)
        # four caches, rotated, so that every call reads its cache from HBM (together more
        # than the 256 MB Infinity Cache at 128K; at 4K and 32K the caches are smaller)
        ncache = 4
        qd = dev.to_device(q)
        ks = [dev.to_device(k) for _ in range(ncache)]
        vs = [dev.to_device(v) for _ in range(ncache)]
        shp = L.gqa_shape(n_q, n_kv, d, ctx)
        ws = torch.empty(L.moe_gqa_decode_workspace_bytes(shp), dtype=torch.uint8, device="cuda")
        out = torch.empty((n_q, d), dtype=torch.int16, device="cuda")
        cur = torch.cuda.current_stream()

        def call(i, stream):
            L.moe_gqa_decode_attention(shp, qd, ks[i % ncache], vs[i % ncache], out, ws,
                                       stream=stream)
        for i in range(8):
            call(i, cur)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(reps):
            call(i, cur)
        torch.cuda.synchronize()
        eager_us = (time.perf_counter() - t0) * 1e6 / reps
        # the same calls as replays of one captured graph of eight (two per cache): the GPU's
        # time per call without the host's launch cost
        per_graph = 2 * ncache
        side = torch.cuda.Stream()
        side.wait_stream(cur)
        with torch.cuda.stream(side):
            for i in range(per_graph):
                call(i, side)
        cur.wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            cap = torch.cuda.current_stream()
            for i in range(per_graph):
                call(i, cap)
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        n_rep = max(1, reps // per_graph)
        t0 = time.perf_counter()
        for _ in range(n_rep):
            g.replay()
        torch.cuda.synchronize()
        us = (time.perf_counter() - t0) * 1e6 / (n_rep * per_graph)
        del g
        nbytes = float(wl.attention_bytes(n_q, n_kv, d, ctx))
        res[name] = {"n_q_heads": n_q, "n_kv_heads": n_kv, "head_dim": d, "ctx": ctx,
                     "us_per_call": us, "eager_us_per_call": eager_us,
                     "algorithmic_bytes": nbytes,
                     "gbs": nbytes / (us * 1e-6) / 1e9,
                     "hbm_frac": nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS,
                     "tokens_per_s_one_layer": 1e6 / us}
        log(f"bench: {name}: {us:.2f} us/call as graph replays ({eager_us:.2f} eager), "
            f"{res[name]['gbs']:.0f} GB/s of cache ({100 * res[name]['hbm_frac']:.1f}% of 8 TB/s)")
        del ks, vs, ws
    return res


def hbm_ceiling(torch, dev):
    """Measured streaming ceiling: a plain device copy of 1 GiB (2 GiB moved) and a streaming
    read of 2 GiB (torch's sum), best of five each, timed with fence-free HIP events."""
    a = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    big = torch.ones(1 << 29, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    e0, e1 = dev.hip_event(), dev.hip_event()

    def best(fn, n=5):
        t = 1e9
        for _ in range(n):
            dev.hip_event_record(e0, stream)
            fn()
            dev.hip_event_record(e1, stream)
            torch.cuda.synchronize()
            t = min(t, dev.hip_elapsed_ms(e0, e1))
        return t

    best(lambda: b.copy_(a), 2)  # warm-up
    t_copy = best(lambda: b.copy_(a))
    t_read = best(lambda: big.sum())
    dev.hip_event_destroy(e0)
    dev.hip_event_destroy(e1)
    copy_gbs = 2 * (1 << 30) / (t_copy * 1e-3) / 1e9
    read_gbs = (1 << 31) / (t_read * 1e-3) / 1e9
    return {"copy_gbs": copy_gbs, "read_gbs": read_gbs, "ceiling_gbs": max(copy_gbs, read_gbs),
            "frac_of_peak": max(copy_gbs, read_gbs) / HBM_PEAK_GBS,
            "method": "torch copy_ of 1 GiB (read + write) and sum over 2 GiB, best of 5, HIP events"}


def sweep(args, torch, L, dev, wl):
    """The grouped gate_up + SwiGLU GEMM of the layer's shape (N = 2F = 1024, K = D = 2048,
    257 groups: 256 experts and the shared one) with n_e rows in every group, for each engine:
    one JSON line per (engine, n_e) with the call's time between two HIP events (it includes
    the tile-map and prepared-copy launches; rocprofv3 gives the GEMM kernel alone), the
    achieved HBM bandwidth on the algorithmic bytes and the achieved bf16 TFLOP/s."""
    cfg = wl.CONFIGS["prefill512"]
    G, N, K = cfg.E + 1, 2 * cfg.F, cfg.D
    w = wl.make_weights(cfg, wl.layer_seed(0))
    q = dev.to_device(w["gate_up_q"])
    sc = dev.to_device(w["gate_up_s"])
    bi = dev.to_device(w["gate_up_b"])
    W = L.q4(q, sc, bi)
    sizes = [int(v) for v in args.sweep_sizes.split(",")]
    stream = torch.cuda.current_stream().cuda_stream
    e0, e1 = dev.hip_event(), dev.hip_event()
    rng = np.random.default_rng(0)
    for n_e in sizes:
        rows = G * n_e
        A = torch.from_numpy(wl.f32_to_bf16_bits(
            rng.standard_normal((rows, K), dtype=np.float32)).view(np.int16)).cuda()
        off = torch.arange(0, rows + 1, n_e, dtype=torch.int32, device="cuda")
        C = torch.empty((rows, N // 2), dtype=torch.int16, device="cuda")
        ws = torch.empty(L.moe_grouped_gemm_q4_workspace_bytes(G, rows, rows, K),
                         dtype=torch.uint8, device="cuda")
        wbytes = G * N * K * 0.5625
        bytes_ = wbytes + rows * K * 2 + rows * (N // 2) * 2
        flops = 2.0 * rows * N * K
        for eng in args.sweep_engines.split(","):
            def call():
                L.moe_grouped_gemm_q4_ex(G, rows, N, K, A, rows, None, off, W, 1, C, ws, eng)
            try:
                for _ in range(3):
                    call()
            except L.MoEError as err:
                log(f"sweep: {eng} n_e={n_e}: {err}")
                continue
            torch.cuda.synchronize()
            reps = max(3, min(20, int(2e5 // max(rows, 1))))
            ts = []
            for _ in range(reps):
                dev.hip_event_record(e0, stream)
                call()
                dev.hip_event_record(e1, stream)
                torch.cuda.synchronize()
                ts.append(dev.hip_elapsed_ms(e0, e1))
            t = float(np.median(ts)) * 1e-3
            rec = {"sweep": "grouped gate_up + SwiGLU, 257 groups, N=1024, K=2048",
                   "engine": eng, "n_e": n_e, "rows": rows, "call_us": t * 1e6,
                   "algorithmic_bytes": bytes_, "gbs": bytes_ / t / 1e9,
                   "hbm_frac": bytes_ / t / 1e9 / HBM_PEAK_GBS,
                   "tflops": flops / t / 1e12, "mfma_frac": flops / t / 1e12 / BF16_PEAK_TFLOPS,
                   "arith_intensity": flops / bytes_}
            print(json.dumps(rec), flush=True)
        del A, C, ws
    dev.hip_event_destroy(e0)
    dev.hip_event_destroy(e1)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (the layer "
              "would shard by tokens, or by experts with an all-to-all of token rows each way)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from bit_grouped_expert_amd import _lib as L
    from bit_grouped_expert_amd import device as dev
    from bit_grouped_expert_amd import workload as wl

    cfg = wl.CONFIGS[args.config]
    assert torch.cuda.is_available()
    L.lib()
    if args.sweep:
        sweep(args, torch, L, dev, wl)
        return
    log(f"bench: config {cfg.name} T={cfg.T} D={cfg.D} E={cfg.E} k={cfg.k} F={cfg.F}")
    host_w0 = None
    sets = []
    for i in range(args.weight_sets):
        w = wl.make_weights(cfg, wl.layer_seed(i))
        if i == 0:
            host_w0 = w
        sets.append(dev.LayerWeights(w, cfg.E))
        log(f"bench: weight set {i} uploaded ({sets[-1].nbytes() / 1e6:.1f} MB)")

    main_res, (x, router) = measure(cfg, sets, args.steps, args.warmup, torch, L, dev, wl)

    secondary = None
    scfg = wl.CONFIGS[SECONDARY]
    if not args.no_secondary and scfg.name != cfg.name and \
            (scfg.D, scfg.E, scfg.F, scfg.bias) == (cfg.D, cfg.E, cfg.F, cfg.bias):
        # same weight sets (the weights do not depend on T), the 8192-token Zipf-routed batch
        s_res, _ = measure(scfg, sets, args.steps, min(args.warmup, 40), torch, L, dev, wl)
        secondary = {"workload": f"{scfg.name}: one MoE layer, T={scfg.T}, Zipf-skewed routing, "
                                 "same shape and weights",
                     "steps": args.steps, "warmup": min(args.warmup, 40), **s_res}

    staged = None
    if not args.no_secondary:
        staged = {"workload": f"{cfg.name} through the staged entry points (route, permute, four "
                              "grouped GEMM calls, combine): offsets kept on the device, and read "
                              "back by the host between the permutation and the GEMMs",
                  "fused_layer_us": main_res["ms_per_step"] * 1e3,
                  **measure_staged(cfg, sets, torch, L, dev, wl)}

    decode = None
    if not args.no_decode:
        decode = {"workload": "decode-sized layers (T=1 and T=4 tokens), same shape and weights: "
                              "the router, then one launch (plan, gate_up, down + combine)"}
        for name in ("decode1", "decode4"):
            dcfg = wl.CONFIGS[name]
            if (dcfg.D, dcfg.E, dcfg.F, dcfg.bias) == (cfg.D, cfg.E, cfg.F, cfg.bias):
                decode[name] = measure_decode(dcfg, sets, torch, L, dev, wl)

    long = None
    lcfg = wl.CONFIGS["long32768"]
    if not args.no_long and (lcfg.D, lcfg.E, lcfg.F, lcfg.bias) == (cfg.D, cfg.E, cfg.F, cfg.bias):
        long = {"workload": "long32768: one MoE layer at T=32768 per weight set, same shape and "
                            "weights, single call vs bounded chunks",
                **measure_long(lcfg, sets, torch, L, dev, wl)}

    attention = None
    if not args.no_attention:
        attention = {"workload": "grouped-query decode attention of the pages' full-attention "
                                 "layers: one query token, 16 query heads on 2 KV heads, head "
                                 "dim 128 (a reading), bf16 KV cache",
                     **measure_attention(torch, L, dev, wl)}

    ceiling = hbm_ceiling(torch, dev)
    log(f"bench: HBM ceiling copy {ceiling['copy_gbs']:.0f} GB/s, read {ceiling['read_gbs']:.0f} GB/s")
    main_res["roofline"]["frac_of_measured_ceiling"] = (
        main_res["roofline"]["achieved"] / ceiling["ceiling_gbs"]
        if main_res["roofline"]["bound"] == "hbm" else None)

    if args.copy_probe:
        # a plain elementwise copy of 1 GiB (torch's vectorized elementwise kernel): the
        # reference for scaling the FETCH_SIZE / WRITE_SIZE counters to bytes
        a = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        torch.mul(a, 1.0, out=b)
        torch.cuda.synchronize()
        log("bench: copy probe (1 GiB elementwise) done")

    cpu = None
    if not args.no_cpu_baseline:
        log("bench: timing the CPU oracle")
        cpu = cpu_baseline(cfg, x, router, host_w0)

    recipe = "bias = -8*scale" if cfg.bias == "neg8" else "bias = -scale*(7.5+0.5z) per group"
    line = {
        "metric": METRIC,
        "value": main_res["value"], "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": main_res["ms_per_step"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded; x ~ N(0,1) bf16, router ~ N(0,0.02) fp32; random int4 codes, "
                f"bf16 scale ~ |N(0,0.02)| per 64, {recipe}; {args.weight_sets} rotating weight sets)",
        "config": {"workload": f"{cfg.name}: one MoE layer, T={cfg.T}, d_model={cfg.D}, "
                               f"{cfg.E} experts top-{cfg.k} + 1 shared, SwiGLU d_ff={cfg.F}, "
                               "int4 g64 bf16 scale+bias",
                   "T": cfg.T, "d_model": cfg.D, "experts": cfg.E, "top_k": cfg.k, "d_ff": cfg.F,
                   "routing": cfg.routing, "parallelism": "single GPU"},
        "stage_us": main_res["stage_us"],
        "latency": main_res["latency"],
        "touched_groups": main_res["touched_groups"],
        "rows_per_group": main_res["rows_per_group"],
        "roofline": main_res["roofline"],
        "layer_roofline": main_res["layer_roofline"],
        "zipf8192": secondary,
        "staged_ablation": staged,
        "decode": decode,
        "long32768": long,
        "gqa_decode_attention": attention,
        "hbm_ceiling": ceiling,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
