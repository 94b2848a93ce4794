"""A hand-built one-expert layer whose MXFP4 blocks use the ends of the E8M0
scale range: byte 0 (2^-127) with zero codes and with nonzero codes (whose
values 0.5, 1, 1.5 times 2^-127 are subnormal), byte 1 (2^-126; code 1 gives
the subnormal 2^-127) and byte 254 (2^127; codes up to 1.5 stay below the
fp32 maximum), next to ordinary bytes.

Activations and intermediates are sized so that every contribution is finite
and no sum cancels: x > 0 everywhere, every code positive, so each output is
a sum of positive terms and its relative error is the arithmetic's alone.
Per 32-column block j of x the magnitude class m_j makes the extreme-scale
weight blocks meet activations that keep their products O(1):

    block 0: x in [2^-126, 2^-125)   (meets gate/up blocks of scale byte 254)
    block 1: x in [2^119, 2^120)     (meets gate/up blocks of scale byte 1)
    block 2: x in [2^120, 2^121)     (meets gate/up blocks of scale byte 0)
    blocks 3-7: x in [1, 2)

The expert's h rows come in four 32-row groups (the down projection's K
blocks): group 0 tiny (~2^-110, meets down blocks of byte 254), group 1 huge
(~2^117, meets byte 1), group 2 huge (~2^119, meets byte 0), group 3 O(1)-O(1e3)
(made by the gate/up blocks of bytes 254, 1, 0 and ordinary ones).  The down
rows cycle through six classes: one extreme block alone (bytes 254, 1, 0),
an ordinary block alone, and two mixes; their other blocks hold zero codes
with scale bytes 0 or 127 (zero codes give exact zeros whatever the scale).

E = 1 and top-1, so the gate is exactly 1 and out = y.  The expected values
come from the oracle (fp64, exact decode); nothing here computes the layer.
"""
from __future__ import annotations

import numpy as np

D, F = 256, 128
X_CLASS = [-126, 119, 120, 0, 0, 0, 0, 0]  # log2 of the lower end of each x block's range


def _set_block(P, S, r, K, b, codes, scale):
    """Row r of a [rows, K] MXFP4 matrix (P [rows][K/2], S [rows][K/32]): block b
    gets the 32 codes and the scale byte."""
    codes = np.asarray(codes, dtype=np.uint8)
    assert codes.shape == (32,) and (codes < 16).all()
    P[r, b * 16:(b + 1) * 16] = codes[0::2] | (codes[1::2] << 4)
    S[r, b] = scale


def build(T: int, seed: int = 3):
    """(x bf16 bits [T, D], router weights fp32 [1, D], packed [1, ...], scales [1, ...])."""
    rng = np.random.default_rng(seed)
    # x: block j in [2^X_CLASS[j], 2^(X_CLASS[j] + 1)), rounded down to bf16
    # (truncating the fp32 bits keeps every value inside its range)
    u = rng.uniform(1.0, 2.0, size=(T, D))
    scale = np.repeat(np.ldexp(1.0, X_CLASS), 32)[None, :]
    x32 = (u * scale).astype(np.float32)
    x = (x32.view(np.uint32) >> 16).astype(np.uint16)
    wr = np.zeros((1, D), dtype=np.float32)
    wr[0, 96:] = 0.01  # the router sees only the ordinary blocks (one expert anyway)

    nb_d, nb_f = D // 32, F // 32
    Pg = np.zeros((F, D // 2), np.uint8)
    Pu = np.zeros((F, D // 2), np.uint8)
    Sg = np.full((F, nb_d), 127, np.uint8)
    Su = np.full((F, nb_d), 127, np.uint8)
    small = lambda n=32: rng.integers(1, 4, size=n)  # codes 1..3: 0.5 .. 1.5
    anyc = lambda: rng.integers(1, 8, size=32)       # codes 1..7: 0.5 .. 6
    for i in range(F):
        a, sub = divmod(i, 32)
        for P, S in ((Pg, Sg), (Pu, Su)):
            # zero-coded blocks keep scale bytes from both ends of the range
            for b in range(nb_d):
                S[i, b] = (0, 254, 127)[(i + b) % 3]
            if a == 0:    # tiny h: ordinary x, scale 2^-64
                for b in range(3, 8):
                    _set_block(P, S, i, D, b, anyc(), 63)
            elif a == 1:  # huge h: ordinary x, scale 2^49
                for b in range(3, 8):
                    _set_block(P, S, i, D, b, anyc(), 176)
            elif a == 2:  # huge h: ordinary x, scale 2^50
                for b in range(3, 8):
                    _set_block(P, S, i, D, b, anyc(), 177)
            else:
                if sub < 8:     # byte 254 against x ~ 2^-126: 8 nonzero codes
                    c = np.zeros(32, np.int64)
                    c[rng.choice(32, 8, replace=False)] = small(8)
                    _set_block(P, S, i, D, 0, c, 254)
                elif sub < 16:  # byte 1 against x ~ 2^119
                    _set_block(P, S, i, D, 1, anyc(), 1)
                elif sub < 24:  # byte 0 (nonzero codes) against x ~ 2^120
                    _set_block(P, S, i, D, 2, anyc(), 0)
                else:           # ordinary blocks and bytes
                    for b in range(3, 8):
                        _set_block(P, S, i, D, b, small(), 121 + b)

    Pd = np.zeros((D, F // 2), np.uint8)
    Sd = np.zeros((D, nb_f), np.uint8)
    for r in range(D):
        cls = r % 6
        for q in range(nb_f):
            Sd[r, q] = (0, 127)[(r + q) % 2]  # zero-coded blocks: bytes 0 and 127
        if cls in (0, 4):
            _set_block(Pd, Sd, r, F, 0, small(), 254)
        if cls in (1, 5):
            _set_block(Pd, Sd, r, F, 1, anyc(), 1)
        if cls in (2, 5):
            _set_block(Pd, Sd, r, F, 2, anyc(), 0)
        if cls == 3:
            _set_block(Pd, Sd, r, F, 3, anyc(), 120)
        if cls == 4:
            _set_block(Pd, Sd, r, F, 3, anyc(), 130)
    packed = np.concatenate([Pg.ravel(), Pu.ravel(), Pd.ravel()])[None, :]
    scales = np.concatenate([Sg.ravel(), Su.ravel(), Sd.ravel()])[None, :]
    return x, wr, packed, scales


def check_design(ref):
    """The oracle's h and out have the magnitudes the design needs: finite,
    positive, and each h group in its range.  ref: oracle result with
    intermediates, T tokens of the one expert (pair p = token p)."""
    h, out = ref.h, ref.out
    assert np.isfinite(h).all() and np.isfinite(out).all()
    assert (h > 0).all() and (out > 0).all()
    lg = np.log2(h)
    assert (lg[:, :32] > -120).all() and (lg[:, :32] < -100).all()
    assert (lg[:, 32:64] > 110).all() and (lg[:, 32:64] < 125).all()
    assert (lg[:, 64:96] > 112).all() and (lg[:, 64:96] < 126).all()
    assert (lg[:, 96:] > -10).all() and (lg[:, 96:] < 20).all()
    return True
