"""Pins of the oracle's router, top-k, permutation, expert FFN and combine.

Each test fixes the oracle to something other than itself: a library routine
(numpy matmul / stable sort, scipy softmax), a hand-worked case whose answer
follows from its construction, an exact invariant of the layer, or the
independent dense brute-force evaluation in oracle/dense_check.py.
"""
import math

import numpy as np
import pytest
from scipy.special import softmax

from oracle import dense_check


def _cfg_inputs(synth_mod, name=None, **kw):
    from dataclasses import replace
    cfg = synth_mod.get_config(name) if name else synth_mod.Config("adhoc", **kw)
    x, wr = synth_mod.routing_inputs(cfg)
    p, s = synth_mod.expert_weights(cfg, nthreads=4)
    return cfg, x, wr, p, s


def _x64(x_bf16):
    return (x_bf16.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# ------------------------------------------------------------------ router / top-k


def test_router_equals_matmul(oracle_mod, synth_mod):
    cfg = synth_mod.Config("r", T=5, d=160, F=32, E=12, k=3)
    x, wr = synth_mod.routing_inputs(cfg)
    ref = _x64(x) @ wr.astype(np.float64).T
    got = oracle_mod.router(x, wr)
    assert np.allclose(got, ref, rtol=1e-13, atol=1e-13)


def test_topk_against_full_sort(oracle_mod):
    rng = np.random.default_rng(0)
    logits = rng.normal(size=(20, 37))
    for k in (1, 2, 5, 37):
        idx, gates, gap = oracle_mod.topk(logits, k)
        for t in range(20):
            order = np.argsort(-logits[t], kind="stable")[:k]
            assert (idx[t] == order).all()
            sel = logits[t, order]
            assert np.allclose(gates[t], softmax(sel), rtol=1e-14, atol=0)
        if k < 37:
            srt = -np.sort(-logits, axis=1)
            assert gap == pytest.approx((srt[:, k - 1] - srt[:, k]).min(), rel=1e-15)
        else:
            assert gap == math.inf


def test_topk_k_equals_E_is_full_softmax(oracle_mod):
    rng = np.random.default_rng(1)
    logits = rng.normal(size=(3, 9)) * 4
    idx, gates, _ = oracle_mod.topk(logits, 9)
    full = softmax(logits, axis=1)
    for t in range(3):
        assert np.allclose(gates[t], full[t, idx[t]], rtol=1e-14)


def test_topk_k1_gate_is_one(oracle_mod):
    rng = np.random.default_rng(2)
    idx, gates, _ = oracle_mod.topk(rng.normal(size=(6, 10)), 1)
    assert (gates == 1.0).all()


def test_topk_tie_break_lower_index(oracle_mod):
    logits = np.array([[1.0, 3.0, 3.0, 2.0], [5.0, 5.0, 5.0, 5.0]])
    idx, gates, gap = oracle_mod.topk(logits, 2)
    assert idx.tolist() == [[1, 2], [0, 1]]
    assert gates[0].tolist() == [0.5, 0.5]
    idx3, _, _ = oracle_mod.topk(logits, 3)
    assert idx3.tolist() == [[1, 2, 3], [0, 1, 2]]


def test_gates_sum_to_one_and_scaling(oracle_mod):
    rng = np.random.default_rng(3)
    logits = rng.normal(size=(16, 64)) * 4
    idx, gates, _ = oracle_mod.topk(logits, 8)
    assert np.allclose(gates.sum(1), 1.0, atol=1e-15)
    # doubling every logit keeps the selection and squares-then-renormalises the gates
    idx2, gates2, _ = oracle_mod.topk(2 * logits, 8)
    assert (idx2 == idx).all()
    sq = gates ** 2
    assert np.allclose(gates2, sq / sq.sum(1, keepdims=True), rtol=1e-12)


# ------------------------------------------------------------------ permutation


def test_permutation_hand_case(oracle_mod):
    idx = np.array([[2, 0], [0, 1]], dtype=np.int32)
    offsets, sslot, pos = oracle_mod.permute(idx, 3)
    assert offsets.tolist() == [0, 2, 3, 4]
    assert sslot.tolist() == [1, 2, 3, 0]
    assert pos.tolist() == [3, 0, 1, 2]


def test_permutation_against_stable_sort(oracle_mod):
    rng = np.random.default_rng(4)
    T, E, k = 50, 23, 5
    idx = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    offsets, sslot, pos = oracle_mod.permute(idx, E)
    flat = idx.reshape(-1)
    ref = np.argsort(flat, kind="stable")  # slots in token-major order, stably by expert
    assert (sslot == ref).all()
    assert (np.sort(sslot) == np.arange(T * k)).all()  # bijection
    assert (pos[sslot] == np.arange(T * k)).all()
    assert offsets[0] == 0 and offsets[-1] == T * k and (np.diff(offsets) >= 0).all()
    assert (np.diff(offsets) == np.bincount(flat, minlength=E)).all()
    toks = sslot // k
    for e in range(E):
        seg = toks[offsets[e]:offsets[e + 1]]
        assert (np.diff(seg) > 0).all()  # token ascending within an expert


# ------------------------------------------------------------------ expert FFN


def _perm_matrix_expert(pi, code, scale_byte, n):
    """Packed [n][n] matrix with one nonzero per row: row i has `code` at column pi[i]."""
    P = np.zeros((n, n // 2), dtype=np.uint8)
    S = np.full((n, n // 32), scale_byte, dtype=np.uint8)
    for i in range(n):
        c = pi[i]
        P[i, c // 2] |= (code if c % 2 == 0 else code << 4)
    return P, S


def test_hand_worked_permutation_expert(oracle_mod):
    # d = F = 32, one expert, one token, k = 1 (gate 1):
    #   gate row i holds 1.0 at column pi[i]   -> g_i = x[pi[i]]
    #   up   row i holds 2.0 at column pi[i]   -> u_i = 2 x[pi[i]]
    #   down row r holds 0.5 at column sg[r]   -> y_r = 0.5 h[sg[r]]
    # so out_r = 0.5 * silu(x[pi[sg[r]]]) * 2 x[pi[sg[r]]] = x_m^2 / (1 + exp(-x_m)), m = pi[sg[r]].
    n = 32
    rng = np.random.default_rng(5)
    pi = rng.permutation(n)
    sg = rng.permutation(n)
    Pg, Sg = _perm_matrix_expert(pi, 2, 127, n)   # code 2 = 1.0
    Pu, Su = _perm_matrix_expert(pi, 4, 127, n)   # code 4 = 2.0
    Pd, Sd = _perm_matrix_expert(sg, 1, 127, n)   # code 1 = 0.5
    packed = np.concatenate([Pg.ravel(), Pu.ravel(), Pd.ravel()])[None, :]
    scales = np.concatenate([Sg.ravel(), Su.ravel(), Sd.ravel()])[None, :]
    xv = np.array([(-1) ** i * (0.25 + i / 8) for i in range(n)], dtype=np.float32)  # bf16-exact
    x = ((xv.view(np.uint32) >> 16).astype(np.uint16))[None, :]
    wr = np.ones((1, n), dtype=np.float32)
    res = oracle_mod.forward(x, wr, packed, scales, k=1, F=n)
    xm = xv.astype(np.float64)[pi[sg]]
    expect = xm * xm / (1.0 + np.exp(-xm))
    assert np.allclose(res.out[0], expect, rtol=1e-15, atol=0)
    assert res.gates[0, 0] == 1.0


def test_single_expert_is_dense_swiglu(oracle_mod, synth_mod):
    # T=1, E=1, k=1: the layer is W_down (silu(W_gate x) * (W_up x)) with numpy matmuls
    cfg = synth_mod.Config("one", T=1, d=96, F=64, E=1, k=1)
    x, wr = synth_mod.routing_inputs(cfg)
    p, s = synth_mod.expert_weights(cfg)
    d, F = cfg.d, cfg.F
    n = F * d
    wg = oracle_mod.dequantize(p[0, : n // 2], s[0, : n // 32], F, d)
    wu = oracle_mod.dequantize(p[0, n // 2: n], s[0, n // 32: n // 16], F, d)
    wd = oracle_mod.dequantize(p[0, n:], s[0, n // 16:], d, F)
    xv = _x64(x)[0]
    g, u = wg @ xv, wu @ xv
    ref = wd @ (g / (1 + np.exp(-g)) * u)
    res = oracle_mod.forward(x, wr, p, s, k=1, F=F)
    assert np.allclose(res.out[0], ref, rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("shape", [
    dict(T=8, d=256, F=128, E=8, k=2),       # the Tiny workload's shape
    dict(T=6, d=512, F=256, E=16, k=4),
    dict(T=3, d=96, F=160, E=5, k=5),        # k = E
    dict(T=7, d=64, F=32, E=11, k=1),
])
def test_oracle_equals_dense_bruteforce(oracle_mod, synth_mod, shape):
    cfg = synth_mod.Config("b", **shape)
    x, wr = synth_mod.routing_inputs(cfg)
    p, s = synth_mod.expert_weights(cfg)
    res = oracle_mod.forward(x, wr, p, s, cfg.k, cfg.F, keep_intermediates=True)
    out, idx, gates, logits = dense_check.dense_forward(x, wr, p, s, cfg.k, cfg.F)
    assert (res.idx == idx).all()
    assert np.allclose(res.gates, gates, rtol=1e-13, atol=1e-15)
    scale = np.abs(out).max()
    assert np.abs(res.out - out).max() <= 1e-12 * scale


def test_tiny_workload_against_dense(oracle_mod, synth_mod):
    cfg, x, wr, p, s = _cfg_inputs(synth_mod, "tiny")
    res = oracle_mod.forward(x, wr, p, s, cfg.k, cfg.F)
    out, idx, gates, _ = dense_check.dense_forward(x, wr, p, s, cfg.k, cfg.F)
    assert (res.idx == idx).all()
    assert np.abs(res.out - out).max() <= 1e-12 * np.abs(out).max()
    assert res.min_gap > 1e-3


# ------------------------------------------------------------------ exact invariants


@pytest.fixture(scope="module")
def small(synth_mod):
    cfg = synth_mod.Config("inv", T=6, d=128, F=96, E=7, k=3)
    x, wr = synth_mod.routing_inputs(cfg)
    p, s = synth_mod.expert_weights(cfg)
    return cfg, x, wr, p, s


def _segments(cfg):
    n = cfg.d * cfg.F
    return dict(gate=slice(0, n // 32), up=slice(n // 32, n // 16), down=slice(n // 16, 3 * n // 32))


def test_down_scale_plus_one_doubles_output(oracle_mod, small):
    cfg, x, wr, p, s = small
    base = oracle_mod.forward(x, wr, p, s, cfg.k, cfg.F).out
    s2 = s.copy()
    s2[:, _segments(cfg)["down"]] += 1
    assert (oracle_mod.forward(x, wr, p, s2, cfg.k, cfg.F).out == 2 * base).all()


def test_up_scale_plus_one_doubles_output(oracle_mod, small):
    cfg, x, wr, p, s = small
    base = oracle_mod.forward(x, wr, p, s, cfg.k, cfg.F).out
    s2 = s.copy()
    s2[:, _segments(cfg)["up"]] += 1
    assert (oracle_mod.forward(x, wr, p, s2, cfg.k, cfg.F).out == 2 * base).all()
    # the gate projection goes through silu, so the same change there is not linear
    s3 = s.copy()
    s3[:, _segments(cfg)["gate"]] += 1
    assert not np.allclose(oracle_mod.forward(x, wr, p, s3, cfg.k, cfg.F).out, 2 * base)


def test_zero_up_codes_give_zero_output(oracle_mod, small):
    cfg, x, wr, p, s = small
    n = cfg.d * cfg.F
    p2 = p.copy()
    p2[:, n // 2: n] = 0
    out = oracle_mod.forward(x, wr, p2, s, cfg.k, cfg.F).out
    assert (out == 0).all()


def test_expert_relabeling_invariance(oracle_mod, small):
    cfg, x, wr, p, s = small
    base = oracle_mod.forward(x, wr, p, s, cfg.k, cfg.F)
    perm = np.random.default_rng(6).permutation(cfg.E)
    res = oracle_mod.forward(x, wr[perm], p[perm], s[perm], cfg.k, cfg.F)
    assert (res.out == base.out).all()
    inv = np.argsort(perm)
    assert (perm[res.idx] == base.idx).all()
    _ = inv


def test_token_permutation_equivariance(oracle_mod, small):
    cfg, x, wr, p, s = small
    base = oracle_mod.forward(x, wr, p, s, cfg.k, cfg.F).out
    perm = np.random.default_rng(7).permutation(cfg.T)
    res = oracle_mod.forward(x[perm], wr, p, s, cfg.k, cfg.F).out
    assert (res == base[perm]).all()


def test_token_mask_matches_full(oracle_mod, small):
    cfg, x, wr, p, s = small
    base = oracle_mod.forward(x, wr, p, s, cfg.k, cfg.F).out
    mask = np.zeros(cfg.T, dtype=np.uint8)
    mask[[1, 4]] = 1
    res = oracle_mod.forward(x, wr, p, s, cfg.k, cfg.F, token_mask=mask).out
    assert (res[[1, 4]] == base[[1, 4]]).all()
    assert (res[[0, 2, 3, 5]] == 0).all()


def test_intermediates_layout(oracle_mod, small):
    cfg, x, wr, p, s = small
    res = oracle_mod.forward(x, wr, p, s, cfg.k, cfg.F, keep_intermediates=True)
    # out[t] = sum_j gate[t, j] * y[pos[t*k + j]]
    recon = np.zeros_like(res.out)
    for t in range(cfg.T):
        for j in range(cfg.k):
            recon[t] += res.gates[t, j] * res.y[res.pos[t * cfg.k + j]]
    assert np.allclose(recon, res.out, rtol=1e-15, atol=0)


def test_empty_batch(oracle_mod, synth_mod):
    cfg = synth_mod.Config("e", T=1, d=64, F=32, E=4, k=2)
    x, wr = synth_mod.routing_inputs(cfg)
    p, s = synth_mod.expert_weights(cfg)
    res = oracle_mod.forward(x[:0], wr, p, s, 2, 32)
    assert res.out.shape == (0, 64)
