"""Dense brute-force evaluation of the MoE layer (numpy, fp64) -- TEST INFRASTRUCTURE.

A second, independent way to compute the layer, used only to pin the C
oracle on small inputs: it decodes every expert's whole matrices with numpy,
runs every token through every expert with matrix products, and only then
keeps the k selected experts per token.  It shares no code with the C oracle
(moe_oracle.c) or the GPU library.  Same readings of the pages as the oracle:
OCP MX E2M1 elements with E8M0 scales of 32-element blocks, even element in
the low nibble, expert bytes gate | up | down, SwiGLU h = silu(Wg x) * (Wu x),
top-k by (logit desc, expert asc), softmax gates over the selected logits.
"""
from __future__ import annotations

import numpy as np


def e2m1_table() -> np.ndarray:
    """Value of each 4-bit code, from its sign / exponent / mantissa fields."""
    codes = np.arange(16)
    sign = np.where(codes & 8, -1.0, 1.0)
    exp_field = (codes >> 1) & 3
    mant = (codes & 1).astype(np.float64)
    mag = np.where(exp_field == 0, mant * 0.5, (1.0 + mant / 2.0) * np.exp2(exp_field - 1.0))
    return sign * mag


def decode_matrix(packed: np.ndarray, scales: np.ndarray, rows: int, K: int) -> np.ndarray:
    """[rows, K/2] nibble bytes + [rows, K/32] E8M0 bytes -> fp64 [rows, K]."""
    p = np.asarray(packed, dtype=np.uint8).reshape(rows, K // 2)
    codes = np.empty((rows, K), dtype=np.uint8)
    codes[:, 0::2] = p & 0x0F
    codes[:, 1::2] = p >> 4
    s = np.asarray(scales, dtype=np.uint8).reshape(rows, K // 32).astype(np.float64)
    scale = np.where(s == 255, np.nan, np.exp2(s - 127.0))
    return e2m1_table()[codes] * np.repeat(scale, 32, axis=1)


def expert_matrices(packed_e: np.ndarray, scales_e: np.ndarray, d: int, F: int):
    n = F * d
    wg = decode_matrix(packed_e[: n // 2], scales_e[: n // 32], F, d)
    wu = decode_matrix(packed_e[n // 2: n], scales_e[n // 32: n // 16], F, d)
    wd = decode_matrix(packed_e[n: 3 * n // 2], scales_e[n // 16: 3 * n // 32], d, F)
    return wg, wu, wd


def dense_forward(x_bf16: np.ndarray, w_r: np.ndarray, packed: np.ndarray, scales: np.ndarray, k: int, F: int):
    """Returns (out [T,d], idx [T,k], gates [T,k], logits [T,E]) in fp64."""
    x = (np.asarray(x_bf16, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    T, d = x.shape
    E = w_r.shape[0]
    logits = x @ np.asarray(w_r, dtype=np.float64).T
    idx = np.empty((T, k), dtype=np.int64)
    gates = np.empty((T, k))
    for t in range(T):
        order = np.lexsort((np.arange(E), -logits[t]))  # logit desc, then expert asc
        sel = order[:k]
        idx[t] = sel
        z = np.exp(logits[t, sel] - logits[t, sel].max())
        gates[t] = z / z.sum()
    # every token through every expert
    ys = np.empty((E, T, d))
    for e in range(E):
        wg, wu, wd = expert_matrices(packed[e], scales[e], d, F)
        g = x @ wg.T
        u = x @ wu.T
        h = g / (1.0 + np.exp(-g)) * u
        ys[e] = h @ wd.T
    out = np.zeros((T, d))
    for t in range(T):
        for j in range(k):
            out[t] += gates[t, j] * ys[idx[t, j], t]
    return out, idx, gates, logits
