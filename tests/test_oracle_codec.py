"""Pins of the oracle's MXFP4 codec against the format's fixed values.

The expected numbers come from tests/golden/mx_format.json (the OCP MX v1.0
code points, written out by hand) or from exact round-trip properties; none
is produced by the code under test.
"""
import json
import math
import os

import numpy as np
import pytest

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "mx_format.json")))


def test_e2m1_all_codes(oracle_mod):
    for code, val in GOLD["e2m1_values"].items():
        if code.startswith("_"):
            continue
        got = oracle_mod.e2m1(int(code))
        assert got == val, (code, got, val)
        assert math.copysign(1.0, got) == math.copysign(1.0, val)  # -0 for code 8


def test_e2m1_symmetry(oracle_mod):
    for c in range(8):
        assert oracle_mod.e2m1(c + 8) == -oracle_mod.e2m1(c)


def test_e8m0_values(oracle_mod):
    for s, val in GOLD["e8m0_values"].items():
        if s.startswith("_"):
            continue
        assert oracle_mod.e8m0(int(s)) == val
    assert math.isnan(oracle_mod.e8m0(255))


def test_bf16_values(oracle_mod):
    for bits, val in GOLD["bf16"].items():
        if bits.startswith("_"):
            continue
        assert oracle_mod.bf16(int(bits)) == val
    # agrees with numpy's reinterpretation for every bit pattern of finite values
    pats = np.arange(0, 65536, 7, dtype=np.uint32)
    with np.errstate(invalid="ignore"):
        ref = (pats << 16).view(np.float32).astype(np.float64)
    for p, r in zip(pats[:2000], ref[:2000]):
        if np.isfinite(r):
            assert oracle_mod.bf16(int(p)) == r


def test_hand_blocks_nibble_order(oracle_mod):
    for hb in GOLD["hand_blocks"]:
        K = hb["K"]
        P = np.zeros((1, K // 2), dtype=np.uint8)
        S = np.full((1, K // 32), 127, dtype=np.uint8)
        P[0, 0] = hb["byte0"]
        S[0, 0] = hb["scale"]
        assert oracle_mod.element(P, S, K, 0, 0) == hb["elem0"]
        assert oracle_mod.element(P, S, K, 0, 1) == hb["elem1"]
        deq = oracle_mod.dequantize(P, S, 1, K)
        assert deq[0, 0] == hb["elem0"] and deq[0, 1] == hb["elem1"]
        assert (deq[0, 2:] == 0).all()


def test_scale_and_row_indexing(oracle_mod):
    # 3 rows x 96 columns: byte for (r, c) at r*48 + c//2, scale at r*3 + c//32
    K, rows = 96, 3
    P = np.zeros((rows, K // 2), dtype=np.uint8)
    S = np.zeros((rows, K // 32), dtype=np.uint8)
    for r in range(rows):
        for b in range(3):
            S[r, b] = 120 + r * 3 + b
    P[2, 33 // 2] = 0x20  # element (2, 33): high nibble -> code 2 = 1.0
    P[1, 64 // 2] = 0x05  # element (1, 64): low nibble -> code 5 = 3.0
    assert oracle_mod.element(P, S, K, 2, 33) == 1.0 * 2.0 ** (120 + 6 + 1 - 127)
    assert oracle_mod.element(P, S, K, 2, 32) == 0.0
    assert oracle_mod.element(P, S, K, 1, 64) == 3.0 * 2.0 ** (120 + 3 + 2 - 127)
    assert oracle_mod.element(P, S, K, 1, 65) == 0.0


def _rne_block(pairs, scale):
    vals = np.zeros(32)
    for i, (v, _) in enumerate(pairs):
        vals[i] = v
    return vals


@pytest.mark.parametrize("key", ["amax4", "amax7_5", "amax_small"])
def test_quantize_rne_and_saturation(oracle_mod, synth_mod, key):
    case = GOLD["rne_cases"][key]
    pairs = case if isinstance(case, list) else case["pairs"]
    scale = 127 if isinstance(case, list) else case["scale"]
    vals = _rne_block(pairs, scale)
    for quant in (oracle_mod.quantize, synth_mod.quantize_mxfp4):
        P, S = quant(vals[None, :])
        assert S[0, 0] == scale, (quant, S[0, 0])
        for i, (_, code) in enumerate(pairs):
            byte = P[0, i // 2]
            got = (byte & 0xF) if i % 2 == 0 else (byte >> 4)
            assert got == code, (quant, key, i, pairs[i], got)


def _representable_rows(rng, rows, K):
    """Rows whose blocks are E2M1 magnitudes times one 2^X, block max in {4, 6}."""
    mags = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    m = rng.choice(mags, size=(rows, K)) * rng.choice([-1.0, 1.0], size=(rows, K))
    m = m.reshape(rows, K // 32, 32)
    top = rng.choice([4.0, 6.0], size=(rows, K // 32)) * rng.choice([-1.0, 1.0], size=(rows, K // 32))
    m[:, :, 0] = top
    X = rng.integers(-20, 10, size=(rows, K // 32, 1))
    return (m * np.exp2(X)).reshape(rows, K), (X[:, :, 0] + 127).astype(np.uint8)


def test_round_trip_exact(oracle_mod, synth_mod):
    rng = np.random.default_rng(1)
    w, s_expect = _representable_rows(rng, 16, 128)
    P, S = oracle_mod.quantize(w)
    assert (S == s_expect).all()
    assert (oracle_mod.dequantize(P, S, 16, 128) == w).all()
    P2, S2 = synth_mod.quantize_mxfp4(w.astype(np.float32))
    assert (P2 == P).all() and (S2 == S).all()


def test_all_zero_block(oracle_mod, synth_mod):
    w = np.zeros((1, 32))
    for quant in (oracle_mod.quantize, synth_mod.quantize_mxfp4):
        P, S = quant(w)
        assert (P == 0).all() and S[0, 0] == 0
    assert (oracle_mod.dequantize(P, S, 1, 32) == 0).all()


def test_quantization_error_bound(oracle_mod):
    # |v - q(v)| <= 2^X (half the widest E2M1 gap, between 4 and 6, is 1),
    # and the block maximum itself is within 2^(X+1) (saturation of (6, 8)).
    rng = np.random.default_rng(2)
    w = rng.normal(0, 0.02, size=(8, 256))
    P, S = oracle_mod.quantize(w)
    deq = oracle_mod.dequantize(P, S, 8, 256)
    step = np.repeat(np.exp2(S.astype(np.float64) - 127), 32, axis=1)
    err = np.abs(deq - w)
    assert (err <= 2 * step).all()
    inner = np.abs(w) <= 6 * step
    assert (err[inner] <= step[inner]).all()


def test_generator_quantizer_matches_oracle(oracle_mod, synth_mod):
    # two independent implementations of the same conversion rule
    rng = np.random.default_rng(3)
    for scale in (0.02, 1.0, 1e-6, 300.0):
        w = (rng.normal(0, scale, size=(32, 224))).astype(np.float32)
        P1, S1 = oracle_mod.quantize(w.astype(np.float64))
        P2, S2 = synth_mod.quantize_mxfp4(w)
        assert (S1 == S2).all() and (P1 == P2).all()
