"""The scale-edge expert (tests/scale_edges.py) does what its GPU parity test
needs: the oracle's h and out are finite and positive, each h group sits in
its designed magnitude range, and the decode of its extreme scale bytes
matches the format's code points (byte 0 = 2^-127, byte 254 = 2^127)."""
import numpy as np

import scale_edges as se


def test_design_ranges(oracle_mod):
    for T in (4, 320):
        x, wr, p, s = se.build(T)
        ref = oracle_mod.forward(x, wr, p, s, 1, se.F, keep_intermediates=True)
        assert se.check_design(ref)
        assert (ref.gates == 1.0).all()


def test_extreme_bytes_present(oracle_mod):
    x, wr, p, s = se.build(4)
    D, F = se.D, se.F
    sg = s[0, : F * D // 32].reshape(F, D // 32)
    sd = s[0, 2 * F * D // 32:].reshape(D, F // 32)
    pg = p[0, : F * D // 2].reshape(F, D // 2)
    # byte 0 with nonzero codes, byte 1, byte 254: in gate/up and in down
    for S, P, K in ((sg, pg, D), (sd, p[0, F * D:].reshape(D, F // 2), F)):
        for byte in (0, 1, 254):
            rows, blocks = np.nonzero(S == byte)
            nz = [(r, b) for r, b in zip(rows, blocks) if P[r, b * 16:(b + 1) * 16].any()]
            assert nz, (byte, K)
            r, b = nz[0]
            w = oracle_mod.dequantize(P[r:r + 1], S[r:r + 1], 1, K)[0, b * 32:(b + 1) * 32]
            codes = np.stack([P[r, b * 16:(b + 1) * 16] & 15, P[r, b * 16:(b + 1) * 16] >> 4], 1).ravel()
            mags = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])[codes & 7]
            assert (w == mags * 2.0 ** (byte - 127)).all()
    # x stays in its blocks' ranges
    xf = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    for j, e in enumerate(se.X_CLASS):
        blk = xf[:, 32 * j: 32 * j + 32]
        assert (blk >= 2.0 ** e).all() and (blk < 2.0 ** (e + 1)).all()
