"""GPU decode of the E8M0 scale range's ends against the oracle: a hand-built
one-expert layer (tests/scale_edges.py) whose blocks use scale bytes 0 (zero
and nonzero codes, subnormal element values), 1 (subnormal for code 1) and
254, on the small-batch path (T = 4, x in LDS, fp32 h) and on the MFMA path
(T = 320).  All terms are positive, so every element can be held to the
layer's 2e-3 bar on its own: |gpu - oracle| <= 2e-3 |oracle| for every
element of h and of out (stricter than the bar's max-normalised form)."""
import numpy as np
import pytest

from helpers import to_device
import scale_edges as se

pytestmark = pytest.mark.gpu

TOL = 2e-3


@pytest.mark.parametrize("T", [4, 320], ids=["small_path", "mfma_path"])
def test_scale_byte_edges(T):
    import torch

    import mxfp4_moe_expert_router_amd as moe
    from oracle import oracle

    print(f"\n[scale-edges] T={T}", flush=True)
    x, wr, p, s = se.build(T)
    ref = oracle.forward(x, wr, p, s, 1, se.F, keep_intermediates=True)
    assert se.check_design(ref)
    xt, wrt, pt, st = to_device(torch, x, wr, p, s)
    dims = moe.LayerDims(T, se.D, se.F, 1)
    ws = moe.alloc_workspace(dims, 1)
    out = moe.forward(xt, wrt, pt, st, 1, workspace=ws, dims=dims)
    torch.cuda.synchronize()
    assert moe.status(ws) == moe.MOE_OK
    h = moe.intermediates(ws, dims, 1)["h"].cpu().numpy().astype(np.float64)
    got = out.cpu().numpy().astype(np.float64)
    eh = np.abs(h - ref.h) / ref.h
    eo = np.abs(got - ref.out) / ref.out
    for g in range(4):
        print(f"[scale-edges] T={T} h group {g}: max rel err {eh[:, 32 * g:32 * g + 32].max():.2e}", flush=True)
    for c in range(6):
        print(f"[scale-edges] T={T} out class {c}: max rel err {eo[:, c::6].max():.2e}", flush=True)
    assert eh.max() <= TOL
    assert eo.max() <= TOL
