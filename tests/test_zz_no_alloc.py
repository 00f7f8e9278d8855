"""moe_layer_forward_noalloc (the entry point for callers that cannot allocate: its workspace
is the library's static per-device scratch array) against moe_layer_forward with a caller
workspace: the same kernels on the same inputs, so every output bit must agree.  Two calls in
a row on the same array, the second with fewer tokens, then a decode-sized third."""
import sys

import numpy as np
import pytest

from bit_grouped_expert_amd import _lib as L
from bit_grouped_expert_amd import device as dev
from bit_grouped_expert_amd import workload as wl

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def test_noalloc_matches_workspace_entry_point():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    L.lib()
    base = wl.CONFIGS["prefill512"]
    lw = dev.LayerWeights(wl.make_weights(base, wl.layer_seed(0)), base.E)
    for T, seed in ((512, 0), (100, 3), (1, 4)):
        cfg = wl.MoEConfig("noalloc", T, base.D, base.E, base.k, base.F)
        say(f"noalloc: T={T} seed={seed}")
        x, router = wl.make_activations(cfg, seed)
        xd, rd = dev.to_device(x), dev.to_device(router)
        shp = L.shape(cfg.T, cfg.D, cfg.E, cfg.k, cfg.F)
        assert L.moe_workspace_bytes(shp) <= L.NOALLOC_SCRATCH_BYTES
        got = torch.full((cfg.T, cfg.D), 0x7FC1, dtype=torch.int16, device="cuda")
        L.moe_layer_forward_noalloc(shp, xd, rd, lw.experts, lw.shared, got)
        torch.cuda.synchronize()
        ws = dev.workspace(shp)
        want = torch.empty_like(got)
        L.moe_layer_forward(shp, xd, rd, lw.experts, lw.shared, want, ws)
        torch.cuda.synchronize()
        g, w = dev.to_host(got, np.uint16), dev.to_host(want, np.uint16)
        assert np.array_equal(g, w), f"T={T}: {int((g != w).sum())} elements differ"
