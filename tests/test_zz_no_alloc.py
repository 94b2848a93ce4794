"""moe_mxfp4_forward_noalloc (the allocation-free entry point, workspace in the
library's own device memory) through the C ABI: the same output, bit for bit,
as moe_mxfp4_forward with a caller workspace, on two calls in a row (the
second with a smaller input), and sizes beyond its 32 MiB workspace are
rejected before anything runs."""
import ctypes

import numpy as np
import pytest

from helpers import OUT_TOL, inputs_for, rel_err, to_device

pytestmark = pytest.mark.gpu


def test_noalloc_matches_forward_twice():
    import torch

    import mxfp4_moe_expert_router_amd as moe
    from oracle import oracle
    from synth import synth

    synth.build()
    oracle.build()
    for shape in (dict(T=8, d=1024, F=512, E=32, k=4), dict(T=3, d=512, F=256, E=16, k=2)):
        cfg = synth.Config("noalloc", **shape)
        print(f"\n[noalloc] T={cfg.T} d={cfg.d} F={cfg.F} E={cfg.E} k={cfg.k}", flush=True)
        x, wr, p, s = inputs_for(synth, cfg)
        xt, wrt, pt, st = to_device(torch, x, wr, p, s)
        dims = moe.LayerDims(cfg.T, cfg.d, cfg.F, cfg.E)
        want = moe.forward(xt, wrt, pt, st, cfg.k, dims=dims)
        got = torch.full((cfg.T, cfg.d), 7.0, dtype=torch.float32, device="cuda")
        moe.forward_noalloc(xt, wrt, pt, st, cfg.k, got, dims=dims)
        torch.cuda.synchronize()
        assert torch.equal(got, want)
        ref = oracle.forward(x, wr, p, s, cfg.k, cfg.F)
        assert rel_err(got.cpu().numpy(), ref.out) <= OUT_TOL


def test_noalloc_rejects_sizes_beyond_its_workspace():
    import mxfp4_moe_expert_router_amd as moe

    lib = moe.binding.lib
    big = moe.LayerDims(64, 7168, 2048, 256)  # workspace over 32 MiB
    assert moe.workspace_bytes(big, 8) > 32 << 20
    D = big.c()
    # valid-looking pointers: the size check comes first, nothing is enqueued
    assert lib.moe_mxfp4_forward_noalloc(ctypes.byref(D), 256, 256, 256, 256, 8, 256, None) == moe.MOE_EWORKSPACE
    ok = moe.LayerDims(32, 7168, 2048, 256)
    assert moe.workspace_bytes(ok, 8) <= 32 << 20
    D = ok.c()
    assert lib.moe_mxfp4_forward_noalloc(ctypes.byref(D), 0, 256, 256, 256, 8, 256, None) == moe.MOE_EINVAL
    assert lib.moe_mxfp4_forward_noalloc(ctypes.byref(D), 264, 256, 256, 256, 8, 256, None) == moe.MOE_EALIGN
