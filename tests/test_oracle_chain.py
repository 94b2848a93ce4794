"""Pins of the oracle's stack of MoE layers on one residual stream
(oracle.forward_layers), of its unit-gain RMS normalisation
(oracle.rms_normalize) and of its bf16 rounding (oracle.round_bf16).

round_bf16 is checked against torch's own fp32 -> bf16 conversion (a library
routine, round to nearest even) and against hand-worked ties;
rms_normalize against torch's rms_norm and closed forms; the stack against
exact properties: one layer is the layer (on the normalised input) plus its
input, a stack whose experts output zero leaves the stream unchanged, the
last layer's contribution is additive and comes from its own weights, and
every layer's input is the library-normalised, library-rounded stream.
"""
import math

import numpy as np
import pytest
import torch


def _x64(x_bf16):
    return (x_bf16.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _torch_norm_bf16_bits(r64, eps=1e-6):
    t = torch.nn.functional.rms_norm(torch.from_numpy(np.asarray(r64, dtype=np.float64)), (r64.shape[-1],), eps=eps)
    return _torch_bf16_bits(t.numpy())


def _torch_bf16_bits(v64):
    t = torch.from_numpy(np.asarray(v64, dtype=np.float64).astype(np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


# ------------------------------------------------------------------ round_bf16


def test_round_bf16_against_torch(oracle_mod):
    rng = np.random.default_rng(11)
    v = np.concatenate([
        rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000),
        # exact fp32 halfway points between two bf16 values: ties
        # (finite: top halves below the all-ones exponent, either sign)
        (((rng.integers(0, 0x7F80, 4000, dtype=np.uint32) | (rng.integers(0, 2, 4000, dtype=np.uint32) << 15))
          << 16) | 0x8000).view(np.float32).astype(np.float64),
        np.array([0.0, -0.0, 1.0, -1.0, 3.0e38, -3.0e38, 1e-40, -1e-42]),
    ])
    v = v[np.isfinite(v.astype(np.float32))]
    assert (oracle_mod.round_bf16(v) == _torch_bf16_bits(v)).all()


def test_round_bf16_hand_ties(oracle_mod):
    # bf16 keeps 8 significand bits: around 1.0 its step is 2^-7
    cases = {
        1.0: 0x3F80,
        1.0 + 2.0 ** -8: 0x3F80,        # halfway, the even neighbour is 1.0
        1.0 + 3 * 2.0 ** -8: 0x3F82,    # halfway between 0x3F81 and 0x3F82: even is 0x3F82
        1.0 + 2.0 ** -8 + 2.0 ** -20: 0x3F81,  # above halfway
        -2.5: 0xC020,
        # first to the nearest fp32 (the 2^-40 is lost), then the tie goes to even
        1.0 + 2.0 ** -8 + 2.0 ** -40: 0x3F80,
    }
    got = oracle_mod.round_bf16(np.array(list(cases)))
    assert [int(g) for g in got] == list(cases.values())


# ------------------------------------------------------------------ rms_normalize


def test_rms_normalize_against_torch(oracle_mod):
    rng = np.random.default_rng(12)
    r = rng.standard_normal((5, 300)) * np.array([[1e-3], [0.5], [1.0], [7.0], [300.0]])
    ref = torch.nn.functional.rms_norm(torch.from_numpy(r), (300,), eps=1e-6).numpy()
    assert np.allclose(oracle_mod.rms_normalize(r), ref, rtol=1e-14, atol=0)


def test_rms_normalize_closed_forms(oracle_mod):
    # a constant row c: c / sqrt(c^2 + eps)
    c = 0.37
    got = oracle_mod.rms_normalize(np.full((1, 64), c))
    assert np.allclose(got, c / math.sqrt(c * c + 1e-6), rtol=1e-15)
    # rows of +-a: mean square a^2
    v = np.array([[3.0, -3.0, 3.0, -3.0]])
    assert np.allclose(oracle_mod.rms_normalize(v, eps=0.0), [[1, -1, 1, -1]], rtol=0, atol=1e-15)
    # a zero row stays zero; the result has unit root mean square (eps -> 0)
    assert (oracle_mod.rms_normalize(np.zeros((1, 8))) == 0).all()
    w = np.random.default_rng(13).standard_normal((3, 100)) * 5
    n = oracle_mod.rms_normalize(w, eps=0.0)
    assert np.allclose(np.sqrt(np.mean(n * n, axis=1)), 1.0, rtol=1e-14)


# ------------------------------------------------------------------ the stack


@pytest.fixture(scope="module")
def stack(synth_mod):
    base = synth_mod.Config("chain", T=6, d=128, F=96, E=7, k=3)
    x, _ = synth_mod.routing_inputs(base)
    wr, p, s = [], [], []
    for l in range(3):
        c = synth_mod.chain_layer_config(base, l)
        wr.append(synth_mod.routing_inputs(c)[1])
        pl, sl = synth_mod.expert_weights(c)
        p.append(pl)
        s.append(sl)
    return base, x, wr, p, s


def test_layers_are_distinct(stack):
    _, _, wr, p, _ = stack
    assert not np.array_equal(wr[0], wr[1]) and not np.array_equal(p[0], p[1])


def test_one_layer_is_input_plus_layer(oracle_mod, stack):
    cfg, x, wr, p, s = stack
    x0 = _torch_norm_bf16_bits(_x64(x))
    one = oracle_mod.forward(x0, wr[0], p[0], s[0], cfg.k, cfg.F)
    res = oracle_mod.forward_layers(x, wr[:1], p[:1], s[:1], cfg.k, cfg.F)
    assert (res.out == _x64(x) + one.out).all()
    assert (res.xs[0] == x0).all()
    assert not (x0 == x).all()  # the normalisation moves the input


def test_zero_expert_output_leaves_stream(oracle_mod, stack):
    cfg, x, wr, p, s = stack
    n = cfg.d * cfg.F
    pz = [q.copy() for q in p]
    for q in pz:
        q[:, n // 2: n] = 0  # up codes 0: h = 0, so every expert returns 0
    res = oracle_mod.forward_layers(x, wr, pz, s, cfg.k, cfg.F)
    assert (res.out == _x64(x)).all()
    assert all((xi == res.xs[0]).all() for xi in res.xs)


def test_last_layer_contribution_is_additive(oracle_mod, stack):
    cfg, x, wr, p, s = stack
    n = cfg.d * cfg.F
    base = oracle_mod.forward_layers(x, wr, p, s, cfg.k, cfg.F)
    s2 = [q.copy() for q in s]
    s2[-1][:, n // 16: 3 * n // 32] += 1  # last layer's down scales x2
    res = oracle_mod.forward_layers(x, wr, p, s2, cfg.k, cfg.F)
    for a, b in zip(base.xs, res.xs):
        assert (a == b).all()  # earlier layers untouched
    last = base.layers[-1].out
    assert np.abs((res.out - base.out) - last).max() <= 1e-12 * np.abs(last).max()
    assert np.abs(last).max() > 0


def test_inputs_are_rounded_stream(oracle_mod, stack):
    cfg, x, wr, p, s = stack
    res = oracle_mod.forward_layers(x, wr, p, s, cfg.k, cfg.F)
    r = _x64(x)
    for l in range(len(wr)):
        assert (res.xs[l] == _torch_norm_bf16_bits(r)).all()
        o = oracle_mod.forward(res.xs[l], wr[l], p[l], s[l], cfg.k, cfg.F)
        assert (o.idx == res.layers[l].idx).all()
        r = r + o.out
    assert (res.out == r).all()
    # the stream really moves the later layers' inputs
    assert not (res.xs[-1] == res.xs[0]).all()
    assert res.min_gap == min(o.min_gap for o in res.layers)


def test_deep_stack_inputs_stay_unit_rms(oracle_mod, synth_mod):
    """Eight layers whose expert outputs are large next to the stream (up
    scales x64, down scales x8): the normalised inputs keep a root mean square
    of 1 (to bf16 rounding) while the stream itself grows."""
    base = synth_mod.Config("deep", T=3, d=64, F=64, E=4, k=2)
    x, _ = synth_mod.routing_inputs(base)
    n = base.d * base.F
    wr, p, s = [], [], []
    for l in range(8):
        c = synth_mod.chain_layer_config(base, l)
        wr.append(synth_mod.routing_inputs(c)[1])
        pl, sl = synth_mod.expert_weights(c)
        sl[:, n // 32: n // 16] += 6
        sl[:, n // 16: 3 * n // 32] += 3
        p.append(pl)
        s.append(sl)
    res = oracle_mod.forward_layers(x, wr, p, s, base.k, base.F)
    assert np.isfinite(res.out).all()
    for xi in res.xs:
        rms = np.sqrt(np.mean(_x64(xi) ** 2, axis=1))
        assert np.allclose(rms, 1.0, atol=1e-2)
    assert np.sqrt(np.mean(res.out ** 2)) > 2 * np.sqrt(np.mean(_x64(x) ** 2))
