"""GPU MXFP4 quantize / pack (moe_mxfp4_quantize) against the oracle's
quantizer, bit for bit: codes and scale bytes.  The oracle quantizer itself is
pinned in test_oracle_codec.py (round trips, RNE ties, saturation, error
bound).  fp32 and bf16 inputs; ragged row counts; hand-built blocks at every
E2M1 decision point (ties go to the even mantissa bit), saturation, zeros of
both signs, fp32 subnormals of both signs and values near the fp32 maximum."""
import numpy as np
import pytest

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


def _gpu(env, w32=None, wbf=None):
    torch, moe, _, _ = env
    if w32 is not None:
        t = torch.from_numpy(np.ascontiguousarray(w32, dtype=np.float32)).cuda()
    else:
        t = torch.from_numpy(np.ascontiguousarray(wbf).view(np.int16)).cuda().view(torch.bfloat16)
    p, s = moe.quantize(t)
    torch.cuda.synchronize()
    return p.cpu().numpy(), s.cpu().numpy()


def _check(env, w32, label):
    _, _, oracle, _ = env
    P, S = oracle.quantize(w32.astype(np.float64))
    p, s = _gpu(env, w32=w32)
    assert (s == S).all(), f"{label}: scale bytes differ at {np.argwhere(s != S)[:4].tolist()}"
    assert (p == P).all(), f"{label}: codes differ at {np.argwhere(p != P)[:4].tolist()}"


@pytest.mark.parametrize("rows,K", [(1, 32), (3, 96), (37, 7168), (129, 2048), (1000, 160)])
def test_random_fp32(env, rows, K):
    _, _, _, synth = env
    w = synth.normals(7, 40, rows, rows * K, 0.02).reshape(rows, K)
    print(f"\n[quant] fp32 rows={rows} K={K}", flush=True)
    _check(env, w, f"fp32 {rows}x{K}")


def test_random_bf16(env):
    _, _, oracle, synth = env
    rows, K = 65, 7168
    w = synth.normals(8, 41, 0, rows * K, 1.0).reshape(rows, K)
    wb = synth.f32_to_bf16(w)
    print("\n[quant] bf16 65x7168", flush=True)
    P, S = oracle.quantize(synth.bf16_to_f32(wb).astype(np.float64))
    p, s = _gpu(env, wbf=wb)
    assert (s == S).all() and (p == P).all()


def test_decision_points_and_edges(env):
    # block b has amax 6 * 2^X (element 0 pins the scale); its other elements
    # sit at, just below and just above every E2M1 decision point
    rows = []
    pts = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 7.0]
    # X from -126 (subnormal decision points) over -121 / -120 (either side of
    # the smallest X the kernel hands to the hardware convert) to 3
    for X in (-126, -121, -120, -10, 0, 3):
        for sgn in (1.0, -1.0):
            row = [6.0 * 2.0 ** X]
            for q in pts:
                for delta in (-1, 0, 1):
                    v = np.nextafter(np.float32(q), np.float32(np.inf if delta > 0 else -np.inf)) if delta else q
                    row.append(sgn * float(v) * 2.0 ** X)
            row += [0.0] * (64 - len(row))
            rows.append(row[:64])
    rows.append([0.0] * 32 + [-0.0] * 32)                                 # zero blocks, both signs
    rows.append([1e-45 * (i % 3) for i in range(64)])                      # fp32 subnormals
    rows.append([-1e-45 * (i % 3) for i in range(32)]                     # negative subnormals, alone
                + [-3e-39 * (i % 5) for i in range(31)] + [2.0 ** -119])   # and under a normal maximum
    rows.append([3.0e38 * ((-1) ** i) for i in range(64)])                # near the fp32 maximum
    rows.append([7.0, -6.5] * 16 + [1.0] + [0.0] * 31)                    # saturation, a lone 1
    w = np.array(rows, dtype=np.float32)
    print(f"\n[quant] {w.shape[0]} hand-built rows", flush=True)
    _check(env, w, "decision points")


def test_device_quantized_weights_feed_the_layer(env):
    """Expert weights prepared on the device (fp32 gate, up and down matrices
    quantized by moe_mxfp4_quantize into the layer's per-expert layout) give
    the layer the same bytes as the oracle's quantizer, and the layer on them
    matches the oracle's layer on the oracle's bytes."""
    torch, moe, oracle, synth = env
    from helpers import OUT_TOL, check_routing, rel_err

    cfg = synth.get_config("tiny")  # its routing seed keeps the top-k gap clear of rounding
    T, d, F, E, k = cfg.T, cfg.d, cfg.F, cfg.E, cfg.k
    x, wr = synth.routing_inputs(cfg)
    print(f"\n[quant] device-quantized experts T={T} d={d} F={F} E={E} k={k}", flush=True)
    packs, scs, ref_p, ref_s = [], [], [], []
    for e in range(E):
        gu = synth.normals(21, 50, e, 2 * F * d, 0.02).reshape(2 * F, d)   # gate rows, then up rows
        dn = synth.normals(21, 51, e, d * F, 0.02).reshape(d, F)
        pg, sg = moe.quantize(torch.from_numpy(gu).cuda())
        pd, sd = moe.quantize(torch.from_numpy(dn).cuda())
        packs.append(torch.cat([pg.reshape(-1), pd.reshape(-1)]))
        scs.append(torch.cat([sg.reshape(-1), sd.reshape(-1)]))
        Pg, Sg = oracle.quantize(gu.astype(np.float64))
        Pd, Sd = oracle.quantize(dn.astype(np.float64))
        ref_p.append(np.concatenate([Pg.ravel(), Pd.ravel()]))
        ref_s.append(np.concatenate([Sg.ravel(), Sd.ravel()]))
    pt, st = torch.stack(packs), torch.stack(scs)
    P, S = np.stack(ref_p), np.stack(ref_s)
    torch.cuda.synchronize()
    assert (pt.cpu().numpy() == P).all() and (st.cpu().numpy() == S).all()
    xt = torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)
    ws = moe.alloc_workspace(moe.LayerDims(T, d, F, E), k)
    out = moe.forward(xt, torch.from_numpy(wr).cuda(), pt, st, k, workspace=ws)
    torch.cuda.synchronize()
    assert moe.status(ws) == moe.MOE_OK
    ref = oracle.forward(x, wr, P, S, k, F)
    assert ref.min_gap > 1e-3
    it = {n: v.cpu().numpy() for n, v in moe.intermediates(ws, moe.LayerDims(T, d, F, E), k).items()}
    check_routing(it["topk_idx"], it["topk_w"], it["offsets"], it["sorted_slot"], ref, k)
    err = rel_err(out.cpu().numpy().astype(np.float64), ref.out)
    print(f"[quant] layer on device-quantized experts: err {err:.2e}", flush=True)
    assert err <= OUT_TOL
