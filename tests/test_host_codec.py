"""The library's host MXFP4 codec (moe_mxfp4_quantize_host,
moe_mxfp4_dequantize_host) through the C ABI, no GPU needed.

Expected values: the format's hand-written code points and rounding cases
(tests/golden/mx_format.json) and the oracle's quantizer / dequantizer, bit
for bit (the library's codec shares no code with the oracle).
"""
import json
import math
import os

import numpy as np
import pytest

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "mx_format.json")))


@pytest.fixture(scope="module")
def moe():
    import mxfp4_moe_expert_router_amd as m
    return m


def _code(P, c):
    b = P[c // 2]
    return int(b & 0xF) if c % 2 == 0 else int(b >> 4)


def _block_of(pairs, filler=0.0):
    v = np.full(32, filler, dtype=np.float32)
    for i, (x, _) in enumerate(pairs):
        v[i] = x
    return v


def test_golden_rounding_cases(moe):
    rc = GOLD["rne_cases"]
    cases = [(rc["amax4"], 127)] + [(rc[k]["pairs"], rc[k]["scale"]) for k in ("amax7_5", "amax_small")]
    for pairs, scale in cases:
        P, S = moe.quantize_host(_block_of(pairs)[None, :])
        assert int(S[0, 0]) == scale
        for i, (x, code) in enumerate(pairs):
            assert _code(P[0], i) == code, (x, _code(P[0], i), code)


def test_golden_decode(moe):
    # every code at scale 127 gives the E2M1 value; the E8M0 bytes give their powers of two
    P = np.array([[c | (c << 4) for c in range(16)]], dtype=np.uint8)  # elements 2c, 2c + 1 hold code c
    S = np.array([[127]], dtype=np.uint8)
    w = moe.dequantize_host(P, S, 1, 32)[0]
    for code, val in GOLD["e2m1_values"].items():
        if code.startswith("_"):
            continue
        c = int(code)
        assert w[2 * c] == val and w[2 * c + 1] == val
        assert math.copysign(1.0, w[2 * c]) == math.copysign(1.0, val)
    for s, val in GOLD["e8m0_values"].items():
        if s.startswith("_"):
            continue
        P1 = np.full((1, 16), 0x22, dtype=np.uint8)  # code 2 = 1.0
        got = moe.dequantize_host(P1, np.array([[int(s)]], np.uint8), 1, 32)[0, 0]
        assert got == np.float32(val)
    assert np.isnan(moe.dequantize_host(np.full((1, 16), 0x22, np.uint8), np.array([[255]], np.uint8), 1, 32)).all()


def test_hand_blocks_nibble_order(moe):
    for hb in GOLD["hand_blocks"]:
        P = np.zeros((1, 16), dtype=np.uint8)
        P[0, 0] = hb["byte0"]
        w = moe.dequantize_host(P, np.array([[hb["scale"]]], np.uint8), 1, 32)[0]
        assert w[0] == hb["elem0"] and w[1] == hb["elem1"]


def test_quantize_equals_oracle_random(moe, oracle_mod):
    rng = np.random.default_rng(5)
    rows, K = 48, 256
    w = (rng.standard_normal((rows, K)) * 0.02).astype(np.float32)
    # block magnitudes over the whole fp32 range, subnormals, zeros, signed zeros
    for r in range(rows):
        for b in range(K // 32):
            e = int(rng.integers(-150, 126))
            w[r, 32 * b: 32 * b + 32] *= np.float32(2.0 ** min(e, 120) * 50)
    w[0, :32] = 0.0
    w[1, :32] = -0.0
    w[2, :32] = np.float32(2.0 ** -149) * rng.integers(-3, 4, 32)
    w[3, :32] = np.float32(3.0e38) * rng.uniform(-1, 1, 32).astype(np.float32)
    w[3, 0] = np.float32(3.4028235e38)
    assert np.isfinite(w).all()
    P, S = moe.quantize_host(w)
    Po, So = oracle_mod.quantize(w.astype(np.float64))
    assert (S == So).all()
    assert (P == Po).all()


def test_quantize_decision_points_equal_oracle(moe, oracle_mod):
    # each midpoint t 2^X of neighbouring E2M1 magnitudes and its fp32 neighbours,
    # with the block maximum fixing X, at X from -127 to 125
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 7.0]
    rows = []
    for X in (-127, -126, -125, -120, -60, -3, 0, 1, 60, 120, 125):
        for t in mids:
            v = np.float32(t * 2.0 ** X)
            if v == 0 or not np.isfinite(v):
                continue
            for cand in (np.nextafter(v, np.float32(0)), v, np.nextafter(v, np.float32(np.inf))):
                blk = np.zeros(32, dtype=np.float32)
                blk[0] = np.float32(4.0 * 2.0 ** X) if X > -127 else np.float32(2.0 ** -125)
                blk[1] = cand
                blk[2] = -cand
                rows.append(blk)
    w = np.stack(rows)
    assert np.isfinite(w).all()
    P, S = moe.quantize_host(w)
    Po, So = oracle_mod.quantize(w.astype(np.float64))
    assert (S == So).all() and (P == Po).all()


def test_dequantize_equals_oracle_every_byte(moe, oracle_mod):
    # all 256 code pairs at the scale bytes of both ends of the range
    for s in (0, 1, 2, 120, 127, 200, 252, 253, 254, 255):
        P = np.arange(256, dtype=np.uint8).reshape(16, 16)
        S = np.full((16, 1), s, dtype=np.uint8)
        got = moe.dequantize_host(P, S, 16, 32)
        with np.errstate(over="ignore", invalid="ignore"):
            ref = oracle_mod.dequantize(P, S, 16, 32).astype(np.float32)
        same = (got == ref) | (np.isnan(got) & np.isnan(ref))
        assert same.all(), s
        assert (np.signbit(got) == np.signbit(ref)).all()


def test_round_trip_of_representable_blocks(moe, oracle_mod):
    # a block whose largest magnitude is 4 or 6 times 2^X and whose other
    # values are E2M1 values times 2^X quantizes back to itself
    rng = np.random.default_rng(9)
    mags = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    rows = []
    for X in (-127, -100, -8, 0, 7, 100, 125):
        for lead in (4.0, 6.0):
            v = rng.choice(mags, 32) * rng.choice([-1, 1], 32)
            v[rng.integers(32)] = lead
            rows.append((v * 2.0 ** X).astype(np.float32))
    w = np.stack(rows)
    P, S = moe.quantize_host(w)
    back = moe.dequantize_host(P, S, w.shape[0], 32)
    assert (back == w).all()


def test_error_codes(moe):
    lib = moe.binding.lib
    w = np.zeros((2, 32), np.float32)
    P = np.zeros((2, 16), np.uint8)
    S = np.zeros((2, 1), np.uint8)
    assert lib.moe_mxfp4_quantize_host(w.ctypes.data, 2, 48, P.ctypes.data, S.ctypes.data) == moe.MOE_ESHAPE
    assert lib.moe_mxfp4_quantize_host(None, 2, 32, P.ctypes.data, S.ctypes.data) == moe.MOE_EINVAL
    assert lib.moe_mxfp4_quantize_host(w.ctypes.data, -1, 32, P.ctypes.data, S.ctypes.data) == moe.MOE_EINVAL
    assert lib.moe_mxfp4_quantize_host(None, 0, 32, None, None) == moe.MOE_OK
    w[1, 5] = np.nan
    P[:] = 0xAB
    assert lib.moe_mxfp4_quantize_host(w.ctypes.data, 2, 32, P.ctypes.data, S.ctypes.data) == moe.MOE_EINVAL
    assert (P == 0xAB).all()  # nothing written
    w[1, 5] = np.inf
    assert lib.moe_mxfp4_quantize_host(w.ctypes.data, 2, 32, P.ctypes.data, S.ctypes.data) == moe.MOE_EINVAL
    out = np.zeros((2, 32), np.float32)
    assert lib.moe_mxfp4_dequantize_host(P.ctypes.data, S.ctypes.data, 2, 40, out.ctypes.data) == moe.MOE_ESHAPE
    assert lib.moe_mxfp4_dequantize_host(P.ctypes.data, None, 2, 32, out.ctypes.data) == moe.MOE_EINVAL
