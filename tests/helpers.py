"""Shared helpers of the GPU parity tests: seeded inputs, device upload,
comparison against the oracle at the layer's tolerances."""
from __future__ import annotations

import numpy as np

OUT_TOL = 2e-3    # max |gpu - oracle| / max |oracle| on the layer output
GATE_TOL = 1e-4   # max |gpu - oracle| on gates (fp32 softmax vs fp64)
INTER_TOL = 2e-3  # same metric as OUT_TOL on h and y, per expert block


def inputs_for(synth, cfg, nthreads=0):
    x, wr = synth.routing_inputs(cfg)
    p, s = synth.expert_weights(cfg, nthreads=nthreads)
    return x, wr, p, s


def to_device(torch, x, wr, p, s, dev="cuda"):
    xt = torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
    return xt, torch.from_numpy(wr).to(dev), torch.from_numpy(p).to(dev), torch.from_numpy(s).to(dev)


def rel_err(got, ref):
    scale = np.abs(ref).max()
    if scale == 0:
        return float(np.abs(got).max())
    return float(np.abs(got.astype(np.float64) - ref).max() / scale)


def check_routing(gpu_idx, gpu_w, gpu_off, gpu_ss, ref, k):
    """Top-k sets, permutation, offsets: bit-exact.  Gates: GATE_TOL."""
    gi = np.asarray(gpu_idx)
    assert (np.sort(gi, axis=1) == np.sort(ref.idx, axis=1)).all(), "top-k sets differ"
    assert (gi == ref.idx).all(), "top-k order differs"
    assert (np.asarray(gpu_off) == ref.offsets).all(), "expert offsets differ"
    assert (np.asarray(gpu_ss) == ref.sorted_slot).all(), "permutation differs"
    gerr = np.abs(np.asarray(gpu_w, dtype=np.float64) - ref.gates).max()
    assert gerr <= GATE_TOL, f"gate error {gerr}"
    return gerr
