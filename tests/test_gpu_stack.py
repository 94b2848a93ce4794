"""GPU parity of a stack of MoE layers on one residual stream
(moe_mxfp4_forward_layers) against the oracle's forward_layers.

Every layer has its own router and expert weights (synth.chain_layer_config).
Compared: the stream's total change out - x against the oracle's r_L - x at
the layer tolerance (the change is what the layers add; x itself is exact);
the last layer's normalised bf16 input against the oracle's (equal but for
rare differences where the value sits on a rounding boundary: the kernel
rounds an fp32 value, the oracle an fp64 one); and the last layer's routing
and permutation bit for bit against the oracle's routing of the input the
kernel actually used (the workspace's inspection copies describe the last
layer).  The one-launch stack and one
launch per layer run the same arithmetic, so their outputs must agree bit for
bit.  Shapes cover the one-launch variants (x of all tokens in LDS with one or
two W_down chunks per lane, and the staged-h variant of one or two tokens) and
the sizes that take one launch per layer (x rows of the workgroup's pairs, the
MFMA path), plus the verify block at full size.
"""
import numpy as np
import pytest

from helpers import OUT_TOL, check_routing, rel_err

pytestmark = pytest.mark.gpu


def _x64(x_bf16):
    return (x_bf16.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _stack_inputs(synth, base, L, nthreads=0):
    x, _ = synth.routing_inputs(base)
    wr, p, s = [], [], []
    for l in range(L):
        c = synth.chain_layer_config(base, l)
        wr.append(synth.routing_inputs(c)[1])
        pl, sl = synth.expert_weights(c, nthreads=nthreads)
        p.append(pl)
        s.append(sl)
    return x, wr, p, s


def _rolled_stack_inputs(synth, base, L, experts):
    """Layer l: its own router weights, and layer 0's experts relabelled
    (expert e of layer l is expert (e + 37 l) mod E of layer 0), so that every
    layer's expert e has its own weights without generating L sets."""
    x, _ = synth.routing_inputs(base)
    p0, s0 = experts
    wr, p, s = [], [], []
    for l in range(L):
        wr.append(synth.routing_inputs(synth.chain_layer_config(base, l))[1])
        p.append(np.roll(p0, -37 * l, axis=0))
        s.append(np.roll(s0, -37 * l, axis=0))
    return x, wr, p, s


def _run_stack(base, L, flags_list, nthreads=0, experts=None):
    import torch

    import mxfp4_moe_expert_router_amd as moe
    from oracle import oracle
    from synth import synth

    oracle.build()
    synth.build()
    print(f"\n[stack] {base.name}: T={base.T} d={base.d} F={base.F} E={base.E} k={base.k} L={L}", flush=True)
    if experts is None:
        x, wr, p, s = _stack_inputs(synth, base, L, nthreads)
    else:
        x, wr, p, s = _rolled_stack_inputs(synth, base, L, experts)
    ref = oracle.forward_layers(x, wr, p, s, base.k, base.F, nthreads=nthreads)
    assert ref.min_gap > 1e-3
    xt = torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)
    wrt = torch.from_numpy(np.stack(wr)).cuda()
    pt = torch.from_numpy(np.stack(p)).cuda()
    st = torch.from_numpy(np.stack(s)).cuda()
    p_last, s_last, wr_last = p[-1], s[-1], wr[-1]
    del p, s
    dims = moe.LayerDims(base.T, base.d, base.F, base.E)
    x64 = _x64(x)
    outs = []
    for flags in flags_list:
        ws = moe.alloc_workspace(dims, base.k)
        out = moe.forward_layers(xt, wrt, pt, st, base.k, workspace=ws, flags=flags, dims=dims)
        torch.cuda.synchronize()
        assert moe.status(ws) == moe.MOE_OK
        it = {k: v.cpu().numpy() for k, v in moe.intermediates(ws, dims, base.k).items()}
        # The last layer's input bf16(rmsnorm(r_{L-1})): the kernel rounds its
        # fp32 value, the oracle its fp64 one (through fp32).  Where the value
        # lies within their difference of a bf16 rounding boundary, the two
        # land on different bf16 values.  So: rare differences, and each
        # kernel value is the rounding of some v' within tau of the oracle's
        # unrounded value (tau = 1e-4 of the largest input; the kernel's fp32
        # stream is off by ~1e-5 absolute, which near zero spans several units
        # of the last place).
        gx = it["x_last"].view(np.uint16)
        ox = ref.xs[L - 1]
        diff = gx != ox
        n_diff = int(diff.sum())
        print(f"[stack] {base.name} flags={flags}: last input bf16 differences {n_diff} of {diff.size}", flush=True)
        assert n_diff <= diff.size // 20
        r_prev = x64 + sum(o.out for o in ref.layers[:-1])
        v = oracle.rms_normalize(r_prev)
        tau = 1e-4 * np.abs(v).max()
        lo = _x64(oracle.round_bf16(v - tau))
        hi = _x64(oracle.round_bf16(v + tau))
        g = _x64(gx)
        assert ((lo <= g) & (g <= hi)).all()
        if n_diff:
            print(f"[stack] {base.name}: largest |kernel x - oracle value| where they differ "
                  f"{np.abs(g - v)[diff].max():.2e} (tau {tau:.2e})", flush=True)
        # the routing the kernel took from its own input: bit for bit
        last_ref = oracle.forward(gx, wr_last, p_last, s_last, base.k, base.F, nthreads=nthreads)
        assert last_ref.min_gap > 1e-3
        check_routing(it["topk_idx"], it["topk_w"], it["offsets"], it["sorted_slot"], last_ref, base.k)
        got = out.cpu().numpy().astype(np.float64)
        err = rel_err(got - x64, ref.out - x64)
        print(f"[stack] {base.name} flags={flags}: change err {err:.2e}", flush=True)
        assert err <= OUT_TOL
        outs.append(out)
        # a second call on the same workspace (tags move on by L) gives the same bits
        out2 = moe.forward_layers(xt, wrt, pt, st, base.k, workspace=ws, flags=flags, dims=dims)
        torch.cuda.synchronize()
        assert moe.status(ws) == moe.MOE_OK
        assert torch.equal(out, out2)
    for o in outs[1:]:
        assert torch.equal(outs[0], o), "one launch and one launch per layer differ"
    return ref


def _cfg(name, **kw):
    from synth import synth
    return synth.Config(name, **kw)


@pytest.mark.parametrize("name,kw,L", [
    ("all_x_T8", dict(T=8, d=256, F=128, E=8, k=2), 3),
    ("all_x_T8_even", dict(T=8, d=256, F=128, E=8, k=2), 4),  # even L: layer 0 writes the workspace buffer
    ("staged_h_T1", dict(T=1, d=512, F=256, E=16, k=4), 4),
    ("two_chunks_T4", dict(T=4, d=256, F=2560, E=8, k=2), 3),
    ("all_x_T9_d7168", dict(T=9, d=7168, F=256, E=32, k=8), 3),
])
def test_one_launch_stack(name, kw, L):
    import mxfp4_moe_expert_router_amd as moe
    assert moe.layers_one_launch(moe.LayerDims(kw["T"], kw["d"], kw["F"], kw["E"]), kw["k"])
    flags = [moe.MOE_LAYERS_ONE_LAUNCH, moe.MOE_LAYERS_PER_LAUNCH]
    if name == "all_x_T8":  # both modes launched cooperatively too: the same bits
        flags += [moe.MOE_LAYERS_ONE_LAUNCH | moe.MOE_LAYERS_COOPERATIVE,
                  moe.MOE_LAYERS_PER_LAUNCH | moe.MOE_LAYERS_COOPERATIVE]
    _run_stack(_cfg(name, **kw), L, flags)


@pytest.mark.parametrize("name,kw,L", [
    ("pairs_T40", dict(T=40, d=4096, F=128, E=16, k=4), 2),
    ("mfma_T128", dict(T=128, d=1024, F=256, E=16, k=4, route_seed=1), 2),
])
def test_per_launch_stack(name, kw, L):
    import mxfp4_moe_expert_router_amd as moe
    assert not moe.layers_one_launch(moe.LayerDims(kw["T"], kw["d"], kw["F"], kw["E"]), kw["k"])
    _run_stack(_cfg(name, **kw), L, [0])


def test_single_layer_stack_is_input_plus_layer():
    """L = 1: out = x + the lone layer's output (moe_mxfp4_forward) on the
    stack's normalised input, bit for bit."""
    import torch

    import mxfp4_moe_expert_router_amd as moe
    from synth import synth

    synth.build()
    base = _cfg("one", T=8, d=256, F=128, E=8, k=2)
    x, wr, p, s = _stack_inputs(synth, base, 1)
    xt = torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)
    wrt, pt, st = (torch.from_numpy(np.stack(a)).cuda() for a in (wr, p, s))
    dims = moe.LayerDims(base.T, base.d, base.F, base.E)
    for flags in (moe.MOE_LAYERS_ONE_LAUNCH, moe.MOE_LAYERS_PER_LAUNCH):
        ws = moe.alloc_workspace(dims, base.k)
        out = moe.forward_layers(xt, wrt, pt, st, base.k, workspace=ws, flags=flags)
        torch.cuda.synchronize()
        x0 = moe.intermediates(ws, dims, base.k)["x_last"].view(torch.bfloat16).clone()
        lone = moe.forward(x0, wrt[0], pt[0], st[0], base.k)
        torch.cuda.synchronize()
        assert torch.equal(out, xt.float() + lone)


def test_verify_stack_full_size(verify_experts):
    """The verify block (T=8, d=7168, ffn=2048, E=256, top-8), three layers
    (own router weights, relabelled experts), both launch modes."""
    import mxfp4_moe_expert_router_amd as moe
    from synth import synth

    base = synth.get_config("verify")
    _run_stack(base, 3, [moe.MOE_LAYERS_ONE_LAUNCH, moe.MOE_LAYERS_PER_LAUNCH], experts=verify_experts)
