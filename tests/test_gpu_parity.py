"""GPU parity of the HIP layer against the CPU oracle, through the C ABI.

Small and ragged shapes (several tiles, ragged chunk / row / token-group
tails), the Tiny workload, hand-worked and degenerate cases, determinism,
the staged (one launch per step) path and the watchdog.  Bars: top-k sets,
order, offsets and permutation bit-exact; gates within 1e-4; output, h and y
within 2e-3 of max |oracle|.
"""
import math
import sys

import numpy as np
import pytest

from helpers import GATE_TOL, INTER_TOL, OUT_TOL, check_routing, inputs_for, rel_err, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch

    import mxfp4_moe_expert_router_amd as moe
    from oracle import oracle
    from synth import synth

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    oracle.build()
    synth.build()
    return torch, moe, oracle, synth


def run_case(env, cfg, staged=False, check_inter=True, x=None, wr=None, p=None, s=None, label=""):
    torch, moe, oracle, synth = env
    print(f"\n[case] {label or cfg.name} T={cfg.T} d={cfg.d} F={cfg.F} E={cfg.E} k={cfg.k} staged={staged}",
          flush=True)
    if x is None:
        x, wr, p, s = inputs_for(synth, cfg)
    ref = oracle.forward(x, wr, p, s, cfg.k, cfg.F, keep_intermediates=check_inter)
    xt, wrt, pt, st = to_device(torch, x, wr, p, s)
    dims = moe.LayerDims(cfg.T, cfg.d, cfg.F, cfg.E)
    ws = moe.alloc_workspace(dims, cfg.k)
    out = moe.forward(xt, wrt, pt, st, cfg.k, workspace=ws, staged=staged, dims=dims)
    torch.cuda.synchronize()
    hdr = ws[:32].view(torch.int32).cpu().numpy()  # header words: status, abort, wait site, index
    st = moe.status(ws)
    assert st == moe.MOE_OK, f"status {st}, watchdog site {hdr[3]} index {hdr[4]}"
    got = out.cpu().numpy()
    it = {k: v.cpu().numpy() for k, v in moe.intermediates(ws, dims, cfg.k).items()}
    check_routing(it["topk_idx"], it["topk_w"], it["offsets"], it["sorted_slot"], ref, cfg.k)
    assert (it["pos"] == ref.pos).all()
    n_act = int((np.diff(ref.offsets) > 0).sum())
    assert int(it["n_active"][0]) == n_act
    act = np.nonzero(np.diff(ref.offsets) > 0)[0]
    assert (it["active"][:n_act] == act).all()
    if check_inter:  # intermediates first: a failure names the step
        for e in act:
            p0, p1 = ref.offsets[e], ref.offsets[e + 1]
            eh = rel_err(it["h"][p0:p1], ref.h[p0:p1])
            assert eh <= INTER_TOL, f"h of expert {e}: {eh}"
        yref = np.empty_like(ref.y)
        for slot in range(cfg.T * cfg.k):
            t, j = divmod(slot, cfg.k)
            yref[slot] = ref.gates[t, j] * ref.y[ref.pos[slot]]
        ey = rel_err(it["y"], yref)
        assert ey <= INTER_TOL, f"y error {ey}"
    err = rel_err(got, ref.out)
    assert err <= OUT_TOL, f"output error {err}"
    print(f"[case] ok: out err {err:.2e}", flush=True)
    return got, ref, it


SMALL = [
    dict(T=1, d=64, F=32, E=4, k=1),
    dict(T=3, d=96, F=160, E=5, k=5),          # k = E, d ragged vs 64-row down tiles
    dict(T=8, d=256, F=128, E=8, k=2),         # Tiny shape
    dict(T=17, d=544, F=96, E=40, k=6),        # 17 chunks per row (< one wave of lanes)
    dict(T=64, d=1056, F=224, E=4, k=2),       # ~32 tokens per expert: many LDS token passes
    dict(T=33, d=2080, F=2080, E=64, k=8),     # 65 chunks per row: second lane pass of one chunk
    dict(T=5, d=7168, F=2048, E=12, k=3),      # full-width experts, few of them
    dict(T=40, d=4096, F=128, E=6, k=2),       # x too large for LDS: each workgroup stages its pairs' rows
    dict(T=48, d=7168, F=64, E=4, k=2),        # ~24 tokens per expert, 10 LDS rows: staged and global x groups
    dict(T=100, d=2048, F=2080, E=16, k=4),    # MFMA path, F % 128 != 0
    dict(T=96, d=1024, F=256, E=4, k=2),       # MFMA path: ~48 tokens per expert, two token passes
    dict(T=100, d=800, F=96, E=3, k=2),        # MFMA path: partial K blocks and partial row units
    dict(T=96, d=800, F=256, E=4, k=2),        # MFMA path: gate/up scales byte by byte, down scales 8 bytes a row
    dict(T=824, d=256, F=128, E=160, k=2),     # MFMA router with 32-token units (520 tiles), the last 24 tokens past T
    dict(T=128, d=256, F=128, E=1024, k=8),    # MFMA path at E = 1024: hundreds of active experts of ~1 token each
]


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "T{T}_d{d}_F{F}_E{E}_k{k}".format(**s))
def test_small_shapes_persistent(env, shape):
    cfg = env[3].Config("small", **shape)
    run_case(env, cfg)


@pytest.mark.parametrize("shape", SMALL[1:5] + SMALL[7:], ids=lambda s: "T{T}_d{d}_F{F}_E{E}_k{k}".format(**s))
def test_small_shapes_staged(env, shape):
    cfg = env[3].Config("small", **shape)
    run_case(env, cfg, staged=True)


MAXIMA = [
    dict(T=4, d=64, F=32, E=1024, k=64),      # E and k at the library's maxima
    dict(T=2, d=8192, F=4096, E=2, k=2),      # d and ffn at the library's maxima
]


@pytest.mark.parametrize("shape", MAXIMA, ids=lambda s: "T{T}_d{d}_F{F}_E{E}_k{k}".format(**s))
def test_maximum_sizes(env, shape):
    """The largest E, top-k, d and ffn the library accepts (include/moe_mxfp4.h)."""
    run_case(env, env[3].Config("max", **shape))


def test_tiny_workload(env):
    cfg = env[3].get_config("tiny")
    run_case(env, cfg)


def _bf16_bits(v):
    return (np.asarray(v, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def test_hand_worked_permutation_expert(env):
    # gate row i = 1.0 at column pi[i], up row i = 2.0 at pi[i], down row r = 0.5 at sg[r]:
    # out_r = x_m^2 / (1 + exp(-x_m)) with m = pi[sg[r]]  (closed form; nibble order,
    # transposition and gate/up roles all matter)
    torch, moe, oracle, synth = env
    n = 64
    rng = np.random.default_rng(11)
    pi, sg = rng.permutation(n), rng.permutation(n)

    def mat(perm, code):
        P = np.zeros((n, n // 2), dtype=np.uint8)
        for i in range(n):
            c = perm[i]
            P[i, c // 2] |= code if c % 2 == 0 else code << 4
        return P.ravel(), np.full(n * n // 32, 127, dtype=np.uint8)

    (pg, sgs), (pu, sus), (pd, sds) = mat(pi, 2), mat(pi, 4), mat(sg, 1)
    packed = np.concatenate([pg, pu, pd])[None, :]
    scales = np.concatenate([sgs, sus, sds])[None, :]
    xv = np.array([(-1) ** i * (0.25 + i / 16) for i in range(n)], dtype=np.float32)
    x = _bf16_bits(xv)[None, :]
    wr = np.ones((1, n), dtype=np.float32)
    xt, wrt, pt, st = to_device(torch, x, wr, packed, scales)
    out = moe.forward(xt, wrt, pt, st, 1).cpu().numpy()[0]
    xm = xv.astype(np.float64)[pi[sg]]
    expect = xm * xm / (1 + np.exp(-xm))
    assert np.abs(out - expect).max() <= 1e-6 * np.abs(expect).max()


def test_all_tokens_same_experts(env):
    # column 0 of x is 1 and W_r[e, 0] is large for e < k: every token picks experts 0..k-1
    torch, moe, oracle, synth = env
    cfg = synth.Config("same", T=24, d=256, F=96, E=16, k=3)
    x, wr, p, s = inputs_for(synth, cfg)
    xf = synth.bf16_to_f32(x).copy()
    xf[:, 0] = 1.0
    x = synth.f32_to_bf16(xf)
    wr = wr.copy()
    wr[:3, 0] = [30.0, 20.0, 10.0]
    got, ref, it = run_case(env, cfg, x=x, wr=wr, p=p, s=s, label="same_experts")
    assert (np.diff(ref.offsets)[:3] == cfg.T).all()


@pytest.mark.parametrize("E,k,tied,label", [
    (16, 4, [2, 5, 9, 12], "four_tied_on_top"),   # the whole top-k is one tie
    (16, 3, [1, 4, 6, 10, 14], "tie_straddles_k"),  # five equal logits, three taken
    (300, 5, [7, 33, 140, 141, 299], "wide_E_tie"),  # more than 256 experts
    (16, 4, None, "all_zero_router"),             # every logit +0: experts 0..k-1
])
def test_tied_logits(env, E, k, tied, label):
    """Equal logits are ordered by expert index (lower first): router rows
    that are exact copies give bit-equal logits on both sides."""
    torch, moe, oracle, synth = env
    cfg = synth.Config(label, T=5, d=256, F=64, E=E, k=k)
    x, wr, p, s = inputs_for(synth, cfg)
    wr = wr.copy()
    if tied is None:
        wr[:] = 0.0
    else:
        xf = synth.bf16_to_f32(x).copy()
        xf[:, 0] = 1.0
        x = synth.f32_to_bf16(xf)
        row = wr[tied[0]].copy()
        row[0] = 40.0  # far above the other logits
        wr[tied] = row
    got, ref, it = run_case(env, cfg, x=x, wr=wr, p=p, s=s, label=label)
    if tied is None:
        assert (ref.idx == np.arange(k)).all()
    else:
        assert (ref.idx[:, :min(k, len(tied))] == np.array(tied[:k])).all()


def test_single_expert_layer(env):
    cfg = env[3].Config("one", T=4, d=320, F=64, E=1, k=1)
    run_case(env, cfg)


def test_empty_batch(env):
    torch, moe, oracle, synth = env
    cfg = synth.Config("empty", T=1, d=64, F=32, E=4, k=2)
    x, wr, p, s = inputs_for(synth, cfg)
    xt, wrt, pt, st = to_device(torch, x[:0], wr, p, s)
    out = moe.forward(xt, wrt, pt, st, 2)
    torch.cuda.synchronize()
    assert out.shape == (0, 64)


def test_deterministic_and_staged_bitwise(env):
    torch, moe, oracle, synth = env
    cfg = synth.Config("det", T=8, d=1024, F=512, E=32, k=4)
    x, wr, p, s = inputs_for(synth, cfg)
    xt, wrt, pt, st = to_device(torch, x, wr, p, s)
    dims = moe.LayerDims(cfg.T, cfg.d, cfg.F, cfg.E)
    ws = moe.alloc_workspace(dims, cfg.k)
    outs = [moe.forward(xt, wrt, pt, st, cfg.k, workspace=ws).clone() for _ in range(5)]
    outs.append(moe.forward(xt, wrt, pt, st, cfg.k, workspace=ws, staged=True).clone())
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o, outs[0])


def test_route_entry_point(env):
    torch, moe, oracle, synth = env
    cfg = synth.Config("route", T=40, d=512, F=64, E=48, k=5)
    x, wr = synth.routing_inputs(cfg)
    logits = oracle.router(x, wr)
    idx, gates, gap = oracle.topk(logits, cfg.k)
    assert gap > 1e-4
    offsets, sslot, pos = oracle.permute(idx, cfg.E)
    xt = torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)
    gi, gw, go, gs = moe.route(xt, torch.from_numpy(wr).cuda(), cfg.k, cfg.F)
    torch.cuda.synchronize()

    class R:
        pass

    r = R()
    r.idx, r.gates, r.offsets, r.sorted_slot = idx, gates, offsets, sslot
    check_routing(gi.cpu().numpy(), gw.cpu().numpy(), go.cpu().numpy(), gs.cpu().numpy(), r, cfg.k)


def test_watchdog_timeout_then_recovery(env):
    # the top-k step waits for router words tagged for a call that never
    # happens: every workgroup hits its 2 ms watchdog, the kernel exits and the
    # status is TIMEOUT; the next normal call on the same workspace works.
    torch, moe, oracle, synth = env
    cfg = synth.get_config("tiny")
    x, wr, p, s = inputs_for(synth, cfg)
    xt, wrt, pt, st = to_device(torch, x, wr, p, s)
    dims = moe.LayerDims(cfg.T, cfg.d, cfg.F, cfg.E)
    ws = moe.alloc_workspace(dims, cfg.k)
    opts = moe.Options(moe.MOE_OPT_WITHHOLD_ARRIVAL, 2000, 0)
    out = torch.zeros((cfg.T, cfg.d), dtype=torch.float32, device="cuda")
    moe.forward(xt, wrt, pt, st, cfg.k, out=out, workspace=ws, options=opts)
    assert moe.status(ws) == moe.MOE_ETIMEOUT
    # no element of out was completed, and none keeps its earlier value: all NaN
    assert torch.isnan(out).all()
    assert moe.status(ws) == moe.MOE_OK  # status is cleared by reading it
    out = moe.forward(xt, wrt, pt, st, cfg.k, out=out, workspace=ws)
    assert moe.status(ws) == moe.MOE_OK
    ref = oracle.forward(x, wr, p, s, cfg.k, cfg.F)
    assert rel_err(out.cpu().numpy(), ref.out) <= OUT_TOL


@pytest.mark.parametrize("shape", [dict(T=8, d=256, F=128, E=8, k=2), dict(T=3, d=512, F=256, E=8, k=3),
                                   dict(T=96, d=1024, F=256, E=4, k=2)],
                         ids=["small_path", "staged_h", "mfma_path"])
def test_withheld_h_leaves_nan_then_recovers(env, shape):
    # the down step waits for h words tagged for a call that never happens:
    # every down wait is abandoned (2 ms), no y is stored, every combine wait is
    # abandoned, so every out element is NaN; status TIMEOUT; the next normal
    # call on the same workspace is correct
    torch, moe, oracle, synth = env
    cfg = synth.Config("hold_h", **shape)
    x, wr, p, s = inputs_for(synth, cfg)
    xt, wrt, pt, st = to_device(torch, x, wr, p, s)
    dims = moe.LayerDims(cfg.T, cfg.d, cfg.F, cfg.E)
    ws = moe.alloc_workspace(dims, cfg.k)
    out = torch.zeros((cfg.T, cfg.d), dtype=torch.float32, device="cuda")
    moe.forward(xt, wrt, pt, st, cfg.k, out=out, workspace=ws, options=moe.Options(moe.MOE_OPT_WITHHOLD_H, 2000, 0))
    assert moe.status(ws) == moe.MOE_ETIMEOUT
    assert torch.isnan(out).all()
    moe.forward(xt, wrt, pt, st, cfg.k, out=out, workspace=ws)
    assert moe.status(ws) == moe.MOE_OK
    ref = oracle.forward(x, wr, p, s, cfg.k, cfg.F)
    assert rel_err(out.cpu().numpy(), ref.out) <= OUT_TOL


ONE_TOKEN = [
    dict(T=1, d=256, F=128, E=8, k=2),        # 4 chunks of ffn: slices of one chunk
    dict(T=1, d=544, F=96, E=40, k=6),        # 3 chunks: three slices per expert, 17 chunks per d row
    dict(T=1, d=800, F=2080, E=16, k=8),      # 65 chunks: 520 one-chunk slices, two per workgroup
    dict(T=1, d=2048, F=1024, E=64, k=8),     # 32 chunks: one-chunk slices, 32 per expert
    dict(T=1, d=512, F=4096, E=16, k=8),      # 128 chunks: four-chunk slices (16 rows per wave load)
]


@pytest.mark.parametrize("shape", ONE_TOKEN, ids=lambda s: "T{T}_d{d}_F{F}_E{E}_k{k}".format(**s))
def test_one_token_kernel(env, shape):
    """One-token layers (decode shapes): every output, h and y against the
    oracle; the same bits with few workgroups (every unit still covered, each
    sum in the same order) and launched cooperatively; the staged path within
    the bar."""
    torch, moe, oracle, synth = env
    cfg = synth.Config("one_tok", **shape)
    got, ref, it = run_case(env, cfg, label="one_token")
    x, wr, p, s = inputs_for(synth, cfg)
    xt, wrt, pt, st = to_device(torch, x, wr, p, s)
    base = moe.forward(xt, wrt, pt, st, cfg.k)
    for g in (1, 3, 37):
        out = moe.forward(xt, wrt, pt, st, cfg.k, options=moe.Options(0, 0, g))
        torch.cuda.synchronize()
        assert torch.equal(out, base), g  # the sums do not depend on the split
    coop = moe.forward(xt, wrt, pt, st, cfg.k, options=moe.Options(moe.MOE_OPT_COOPERATIVE, 0, 0))
    staged = moe.forward(xt, wrt, pt, st, cfg.k, staged=True)
    torch.cuda.synchronize()
    assert torch.equal(coop, base)
    assert rel_err(staged.cpu().numpy(), ref.out) <= OUT_TOL


def test_one_token_watchdog(env):
    # a one-token layer's top-k wait abandoned: all NaN, status TIMEOUT, then a
    # normal call on the same workspace
    torch, moe, oracle, synth = env
    cfg = synth.Config("one_tok_hold", T=1, d=256, F=128, E=8, k=2)
    x, wr, p, s = inputs_for(synth, cfg)
    xt, wrt, pt, st = to_device(torch, x, wr, p, s)
    dims = moe.LayerDims(cfg.T, cfg.d, cfg.F, cfg.E)
    ws = moe.alloc_workspace(dims, cfg.k)
    out = torch.zeros((cfg.T, cfg.d), dtype=torch.float32, device="cuda")
    moe.forward(xt, wrt, pt, st, cfg.k, out=out, workspace=ws, options=moe.Options(moe.MOE_OPT_WITHHOLD_ARRIVAL, 2000, 0))
    assert moe.status(ws) == moe.MOE_ETIMEOUT
    assert torch.isnan(out).all()
    moe.forward(xt, wrt, pt, st, cfg.k, out=out, workspace=ws)
    assert moe.status(ws) == moe.MOE_OK
    ref = oracle.forward(x, wr, p, s, cfg.k, cfg.F)
    assert rel_err(out.cpu().numpy(), ref.out) <= OUT_TOL


def test_small_grid_option(env):
    # a persistent launch with only a few workgroups still covers every unit
    torch, moe, oracle, synth = env
    cfg = synth.Config("grid", T=8, d=512, F=256, E=16, k=4)
    x, wr, p, s = inputs_for(synth, cfg)
    ref = oracle.forward(x, wr, p, s, cfg.k, cfg.F)
    xt, wrt, pt, st = to_device(torch, x, wr, p, s)
    for g in (1, 3, 37):
        out = moe.forward(xt, wrt, pt, st, cfg.k, options=moe.Options(0, 0, g))
        torch.cuda.synchronize()
        assert rel_err(out.cpu().numpy(), ref.out) <= OUT_TOL, g


def test_mfma_grid_options(env):
    """MFMA path (both router splits) on grids of 1, 3, 37, 40, 64 and 100 workgroups: one chunk
    for the whole grid (37, 100: not a multiple of 8), 5 and 8 workgroups per
    XCD chunk (40, 64), more than 64 per chunk (100: down units dealt by index
    instead of by gate/up work).  Every grid covers every unit once: the
    output matches the oracle and, as a unit computes the same values on
    whichever workgroup runs it, equals the default grid's bit for bit."""
    torch, moe, oracle, synth = env
    # the router splits K in two (16 tiles), then takes 32-token units (520 tiles)
    for shape in (dict(T=100, d=2048, F=2080, E=16, k=4), dict(T=824, d=256, F=128, E=160, k=2)):
        cfg = synth.Config("mfma_grid", **shape)
        x, wr, p, s = inputs_for(synth, cfg)
        ref = oracle.forward(x, wr, p, s, cfg.k, cfg.F)
        xt, wrt, pt, st = to_device(torch, x, wr, p, s)
        base = moe.forward(xt, wrt, pt, st, cfg.k).cpu().numpy()
        assert rel_err(base, ref.out) <= OUT_TOL
        for g in (1, 3, 37, 40, 64, 100):
            print(f"[case] mfma T={cfg.T} grid {g}", flush=True)
            out = moe.forward(xt, wrt, pt, st, cfg.k, options=moe.Options(0, 0, g))
            torch.cuda.synchronize()
            got = out.cpu().numpy()
            assert np.array_equal(got.view(np.uint32), base.view(np.uint32)), (cfg.T, g)


def test_cooperative_launch_option(env):
    # the cooperative launch gives the same bits as the default plain launch
    torch, moe, oracle, synth = env
    cfg = synth.Config("coop", T=8, d=512, F=256, E=16, k=4)
    x, wr, p, s = inputs_for(synth, cfg)
    xt, wrt, pt, st = to_device(torch, x, wr, p, s)
    a = moe.forward(xt, wrt, pt, st, cfg.k)
    b = moe.forward(xt, wrt, pt, st, cfg.k, options=moe.Options(moe.MOE_OPT_COOPERATIVE, 0, 0))
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    ref = oracle.forward(x, wr, p, s, cfg.k, cfg.F)
    assert rel_err(b.cpu().numpy(), ref.out) <= OUT_TOL
