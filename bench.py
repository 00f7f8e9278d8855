#!/usr/bin/env python3
"""MoE-layer throughput on one MI355X.

A step is one moe_layer_forward (routing, histogram/scan/scatter, grouped gate_up +
SwiGLU, grouped down, weighted combine) over one batch of synthetic tokens whose
inputs are resident in HBM.  The default workload is the 512-token prefill of a
Qwen3.6-35B-A3B-shaped layer (d_model 2048, 256 experts top-8 + 1 shared expert,
d_ff 512, int4 weights with bf16 scale and bias per 64).  Four distinct weight sets
(455 MB each, more than the 256 MB Infinity Cache) rotate so that every step streams
its weights from HBM.

Prints one JSON line: value = tokens/s, plus the roofline of the dominant kernel
(grouped gate_up, timed inside the timed region with two HIP events that the library
records on the layer's stream just before and just after that stage; the events are
created without the system-scope fence of a default event) and the CPU
oracle's rate on a bounded sample.  The per-stage breakdown (stage_us) comes from a
separate pass after the timed region with an event at every stage boundary, since those
events themselves cost a few microseconds per step.

    python bench.py [--steps K] [--warmup W] [--config prefill512|zipf8192|...]
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

# the gate_up kernel the library picks for each workload (engine chosen by group size)
KERNEL_LABEL = {
    "prefill512": "grouped gate_up + SwiGLU (q4_resident_kernel<true, 4>)",
    "decode1": "grouped gate_up + SwiGLU (q4_resident_kernel<true, 4>)",
    "decode4": "grouped gate_up + SwiGLU (q4_resident_kernel<true, 4>)",
    "uniform8192": "grouped gate_up + SwiGLU (q4_wide_kernel<true>)",
    "zipf8192": "grouped gate_up + SwiGLU (q4_wide_kernel<true>)",
    "long32768": "grouped gate_up + SwiGLU (q4_wide_kernel<true>)",
}

# counters of a plain copy kernel of known size, read in the same rocprofv3 --pmc runs
# as the gate_up kernel (KiB per dispatch); None until profiled
TRAFFIC = {
    # rocprofv3 --pmc FETCH_SIZE, then WRITE_SIZE, over `bench.py --config prefill512 --steps 2
    # --warmup 1 --no-cpu-baseline --copy-probe` (summary in profiles/)
    "prefill512": {"fetch_kib": 172137.6, "write_kib": 4609.0,
                   "copy_fetch_kib": 524325.2, "copy_write_kib": 1048576.0, "copy_bytes": 2 ** 30},
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--config", default="prefill512")
    ap.add_argument("--weight-sets", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run one plain 1 GiB device copy (for scaling PMC byte counters)")
    return ap.parse_args()


def gate_up_algorithmic(cfg, touched_groups):
    """Bytes and flops the grouped gate_up must move/do at minimum: touched groups' codes +
    scale + bias (2F x D weights at 0.5625 B each), x read once, activations written."""
    wbytes = touched_groups * 2 * cfg.F * cfg.D * (4 + 32 / 64) / 8
    bytes_ = wbytes + cfg.T * cfg.D * 2 + (cfg.k + 1) * cfg.T * cfg.F * 2
    flops = 2.0 * (cfg.k + 1) * cfg.T * 2 * cfg.F * cfg.D
    return bytes_, flops


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
    return {"value": n / dt, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": sample, "seconds": round(dt, 3)}


_HIP = None
HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000  # hipEventDisableSystemFence


def _hip():
    """The HIP runtime that torch has already loaded (for timing events only)."""
    global _HIP
    if _HIP is None:
        import ctypes
        _HIP = ctypes.CDLL("libamdhip64.so")
    return _HIP


def hip_event() -> int:
    """A timing HIP event without the system-scope fence on completion (raw handle)."""
    import ctypes
    e = ctypes.c_void_p()
    rc = _hip().hipEventCreateWithFlags(ctypes.byref(e), ctypes.c_uint(HIP_EVENT_DISABLE_SYSTEM_FENCE))
    if rc != 0:
        raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
    return e.value


def hip_elapsed_ms(a: int, b: int) -> float:
    import ctypes
    ms = ctypes.c_float()
    rc = _hip().hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b))
    if rc != 0:
        raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
    return ms.value


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the layer would shard by tokens or experts; see the design notes)", file=sys.stderr)
        sys.exit(2)

    import torch
    from bit_grouped_expert_amd import _lib as L
    from bit_grouped_expert_amd import device as dev
    from bit_grouped_expert_amd import workload as wl

    cfg = wl.CONFIGS[args.config]
    assert torch.cuda.is_available()
    L.lib()
    log(f"bench: config {cfg.name} T={cfg.T} D={cfg.D} E={cfg.E} k={cfg.k} F={cfg.F}")
    x, router = wl.make_activations(cfg, 0)
    host_w0 = None
    sets = []
    for i in range(args.weight_sets):
        w = wl.make_weights(cfg, wl.layer_seed(i))
        if i == 0:
            host_w0 = w
        sets.append(dev.LayerWeights(w, cfg.E))
        log(f"bench: weight set {i} uploaded ({sets[-1].nbytes() / 1e6:.1f} MB)")
    xd, rd = dev.to_device(x), dev.to_device(router)
    shp = L.shape(cfg.T, cfg.D, cfg.E, cfg.k, cfg.F)
    ws = dev.workspace(shp)
    out = torch.empty((cfg.T, cfg.D), dtype=torch.int16, device="cuda")
    stream = torch.cuda.current_stream()

    def step(i):
        lw = sets[i % len(sets)]
        L.moe_layer_forward(shp, xd, rd, lw.experts, lw.shared, out, ws, stream=stream)

    # HIP events that the library records on the layer's stream.  They are created without
    # the system-scope fence that a default event performs when it completes (a cache
    # write-back and invalidate that slows the work after it): these events only time.
    # In the timed steps only the two events that bracket the gate_up stage are passed;
    # the breakdown pass after the timed region passes all of them.
    nst = L.N_STAGE_EVENTS
    GU = 2  # events[2]: after the permutation, events[3]: after gate_up
    n_brk = min(args.steps, 20)
    evs = [[hip_event() for _ in range(nst)] for _ in range(args.steps)]
    brk = [[hip_event() for _ in range(nst)] for _ in range(n_brk)]

    def step_events(i, row, only_gate_up):
        lw = sets[i % len(sets)]
        if only_gate_up:
            row = [e if j in (GU, GU + 1) else None for j, e in enumerate(row)]
        L.moe_layer_forward_events(shp, xd, rd, lw.experts, lw.shared, out, ws, row,
                                   stream=stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    log(f"bench: warmup done ({args.warmup} steps)")

    # ---- timed region: exactly K steps, each with the two gate_up events
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step_events(i, evs[i], True)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps
    log(f"bench: {args.steps} steps in {elapsed * 1e3:.2f} ms")
    gu_ms = float(np.mean([hip_elapsed_ms(evs[i][GU], evs[i][GU + 1]) for i in range(args.steps)]))

    # ---- per-stage breakdown (reporting only, outside the timed region)
    for i in range(n_brk):
        step_events(i, brk[i], False)
    torch.cuda.synchronize()
    names = ["route", "permute", "gate_up", "down", "combine"]
    stage_ms = {n: float(np.mean([hip_elapsed_ms(brk[i][j], brk[i][j + 1]) for i in range(n_brk)]))
                for j, n in enumerate(names)}
    log(f"bench: gate_up {gu_ms * 1e3:.1f}us in the timed steps; breakdown pass (events at "
        "every stage): " + ", ".join(f"{k}={v * 1e3:.1f}us" for k, v in stage_ms.items()))

    # touched groups from this run's own group offsets (reporting only)
    lay = L.moe_workspace_layout(shp)
    offs = ws[lay.offsets:lay.offsets + 4 * (cfg.E + 2)].cpu().numpy().view(np.int32)
    touched = int(np.count_nonzero(np.diff(offs[:cfg.E + 1]))) + 1
    gb, gf = gate_up_algorithmic(cfg, touched)
    gu_s = gu_ms * 1e-3
    if gf / gb < RIDGE:
        roof = {"bound": "hbm", "achieved": gb / gu_s / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": gf / gu_s / 1e12, "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    t = TRAFFIC.get(cfg.name)
    if t:
        scale_f = t["copy_bytes"] / (t["copy_fetch_kib"] * 1024)
        scale_w = t["copy_bytes"] / (t["copy_write_kib"] * 1024)
        roof["traffic"] = t["fetch_kib"] * 1024 * scale_f + t["write_kib"] * 1024 * scale_w
    else:
        roof["traffic"] = None
    roof["kernel"] = KERNEL_LABEL.get(cfg.name, "grouped gate_up + SwiGLU")
    roof["algorithmic_bytes"] = gb
    roof["algorithmic_flops"] = gf
    roof["kernel_us"] = gu_s * 1e6

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

    value = cfg.T / (ms_per_step * 1e-3)
    line = {
        "metric": "MoE-layer tokens/sec (T=512 prefill; % of HBM / MFMA roofline)",
        "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded; random-init int4-g64 weights, 4 rotating weight sets)",
        "config": {"workload": f"{cfg.name}: one MoE layer, T={cfg.T}, d_model={cfg.D}, "
                               f"{cfg.E} experts top-{cfg.k} + 1 shared, SwiGLU d_ff={cfg.F}, "
                               "int4 g64 bf16 scale+bias",
                   "T": cfg.T, "d_model": cfg.D, "experts": cfg.E, "top_k": cfg.k, "d_ff": cfg.F,
                   "routing": cfg.routing, "parallelism": "single GPU"},
        "stage_us": {k: v * 1e3 for k, v in stage_ms.items()},
        "touched_groups": touched,
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
