"""Python access to the CPU oracle (moe_oracle.c) -- TEST INFRASTRUCTURE.

Only the tests, the package's smoke check and the benchmark's CPU-baseline leg
may import this module.  It compiles moe_oracle.c with gcc (OpenMP) into
liboracle.so next to it and wraps the C functions for numpy arrays.  Nothing
here touches the GPU library.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")


def build(force: bool = False) -> str:
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", _SRC, "-o", tmp, "-lm"],
                       check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _L():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        vp, i32, i64, u32, dbl = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_uint, ctypes.c_double
        lib.oracle_e2m1.restype = dbl
        lib.oracle_e2m1.argtypes = [u32]
        lib.oracle_e8m0.restype = dbl
        lib.oracle_e8m0.argtypes = [u32]
        lib.oracle_bf16.restype = dbl
        lib.oracle_bf16.argtypes = [ctypes.c_uint16]
        lib.oracle_mxfp4_element.restype = dbl
        lib.oracle_mxfp4_element.argtypes = [vp, vp, i64, i64, i64]
        lib.oracle_dequantize.restype = None
        lib.oracle_dequantize.argtypes = [vp, vp, i64, i64, vp]
        lib.oracle_quantize.restype = None
        lib.oracle_quantize.argtypes = [vp, i64, i64, vp, vp]
        lib.oracle_router.restype = None
        lib.oracle_router.argtypes = [vp, vp, i32, i32, i32, vp]
        lib.oracle_topk.restype = dbl
        lib.oracle_topk.argtypes = [vp, i32, i32, i32, vp, vp]
        lib.oracle_permute.restype = None
        lib.oracle_permute.argtypes = [vp, i32, i32, i32, vp, vp, vp]
        lib.oracle_silu.restype = dbl
        lib.oracle_silu.argtypes = [dbl]
        lib.oracle_forward.restype = dbl
        lib.oracle_forward.argtypes = [i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp, vp,
                                       vp, vp, vp, vp]
        _lib = lib
    return _lib


def _p(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data


def e2m1(code: int) -> float:
    return float(_L().oracle_e2m1(code))


def e8m0(s: int) -> float:
    return float(_L().oracle_e8m0(s))


def bf16(bits: int) -> float:
    return float(_L().oracle_bf16(bits))


def silu(z: float) -> float:
    return float(_L().oracle_silu(z))


def element(packed: np.ndarray, scales: np.ndarray, K: int, r: int, c: int) -> float:
    return float(_L().oracle_mxfp4_element(_p(packed), _p(scales), K, r, c))


def dequantize(packed: np.ndarray, scales: np.ndarray, rows: int, K: int) -> np.ndarray:
    out = np.empty((rows, K), dtype=np.float64)
    _L().oracle_dequantize(_p(np.ascontiguousarray(packed)), _p(np.ascontiguousarray(scales)), rows, K, _p(out))
    return out


def quantize(w: np.ndarray):
    w = np.ascontiguousarray(w, dtype=np.float64)
    rows, K = w.shape
    P = np.zeros((rows, K // 2), dtype=np.uint8)
    S = np.zeros((rows, K // 32), dtype=np.uint8)
    _L().oracle_quantize(_p(w), rows, K, _p(P), _p(S))
    return P, S


def router(x_bf16: np.ndarray, w_r: np.ndarray) -> np.ndarray:
    x_bf16 = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    w_r = np.ascontiguousarray(w_r, dtype=np.float32)
    T, d = x_bf16.shape
    E = w_r.shape[0]
    out = np.empty((T, E), dtype=np.float64)
    _L().oracle_router(_p(x_bf16), _p(w_r), T, d, E, _p(out))
    return out


def topk(logits: np.ndarray, k: int):
    logits = np.ascontiguousarray(logits, dtype=np.float64)
    T, E = logits.shape
    idx = np.empty((T, k), dtype=np.int32)
    gates = np.empty((T, k), dtype=np.float64)
    gap = _L().oracle_topk(_p(logits), T, E, k, _p(idx), _p(gates))
    return idx, gates, float(gap)


def permute(idx: np.ndarray, E: int):
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    T, k = idx.shape
    offsets = np.empty(E + 1, dtype=np.int32)
    sslot = np.empty(T * k, dtype=np.int32)
    pos = np.empty(T * k, dtype=np.int32)
    _L().oracle_permute(_p(idx), T, E, k, _p(offsets), _p(sslot), _p(pos))
    return offsets, sslot, pos


@dataclass
class OracleResult:
    out: np.ndarray  # fp64 [T, d]
    logits: np.ndarray  # fp64 [T, E]
    idx: np.ndarray  # int32 [T, k]
    gates: np.ndarray  # fp64 [T, k]
    offsets: np.ndarray  # int32 [E+1]
    sorted_slot: np.ndarray  # int32 [T*k]
    pos: np.ndarray  # int32 [T*k]
    h: Optional[np.ndarray]  # fp64 [T*k, F], pair order
    y: Optional[np.ndarray]  # fp64 [T*k, d], pair order
    min_gap: float


def forward(x_bf16: np.ndarray, w_r: np.ndarray, packed: np.ndarray, scales: np.ndarray, k: int, F: int,
            token_mask: Optional[np.ndarray] = None, nthreads: int = 0,
            keep_intermediates: bool = False) -> OracleResult:
    """The whole layer in fp64.  packed: [E, 3dF/2] uint8, scales: [E, 3dF/32]."""
    x_bf16 = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    w_r = np.ascontiguousarray(w_r, dtype=np.float32)
    T, d = x_bf16.shape
    E = w_r.shape[0]
    assert packed.shape[0] == E and scales.shape[0] == E
    assert packed.shape[1] == 3 * d * F // 2 and scales.shape[1] == 3 * d * F // 32
    packed = np.ascontiguousarray(packed)
    scales = np.ascontiguousarray(scales)
    out = np.zeros((T, d), dtype=np.float64)
    logits = np.empty((T, E), dtype=np.float64)
    idx = np.empty((T, k), dtype=np.int32)
    gates = np.empty((T, k), dtype=np.float64)
    offsets = np.empty(E + 1, dtype=np.int32)
    sslot = np.empty(T * k, dtype=np.int32)
    pos = np.empty(T * k, dtype=np.int32)
    h = np.zeros((T * k, F), dtype=np.float64) if keep_intermediates else None
    y = np.zeros((T * k, d), dtype=np.float64) if keep_intermediates else None
    mask = None
    if token_mask is not None:
        mask = np.ascontiguousarray(token_mask, dtype=np.uint8)
        assert mask.shape == (T,)
    if nthreads <= 0:
        nthreads = min(16, os.cpu_count() or 1)
    gap = _L().oracle_forward(T, d, F, E, k, _p(x_bf16), _p(w_r), _p(packed), _p(scales), _p(mask), nthreads,
                              _p(out), _p(logits), _p(idx), _p(gates), _p(offsets), _p(sslot), _p(pos), _p(h),
                              _p(y))
    if np.isnan(gap):
        raise ValueError("oracle_forward rejected its arguments")
    return OracleResult(out, logits, idx, gates, offsets, sslot, pos, h, y, float(gap))


def round_bf16(v: np.ndarray) -> np.ndarray:
    """fp64 values -> bf16 bit patterns: first to the nearest fp32 (numpy's
    cast, ties to even), then to the nearest bf16, ties to the even last kept
    bit (bf16 is the top half of a binary32).  Finite inputs."""
    f = np.ascontiguousarray(v, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = (u + 0x7FFF + lsb) >> 16
    return r.astype(np.uint16)


@dataclass
class ChainResult:
    out: np.ndarray          # r_L, fp64 [T, d]
    layers: list             # OracleResult of every layer
    xs: list                 # x_l (bf16 bit patterns, normalised) fed to layer l
    min_gap: float           # smallest top-k gap over all layers


STACK_EPS = 1e-6


def rms_normalize(r: np.ndarray, eps: float = STACK_EPS) -> np.ndarray:
    """Unit-gain RMS normalisation of each row: v / sqrt(mean(v^2) + eps), fp64."""
    r = np.asarray(r, dtype=np.float64)
    return r / np.sqrt(np.mean(r * r, axis=-1, keepdims=True) + eps)


def forward_layers(x_bf16: np.ndarray, w_r: list, packed: list, scales: list, k: int, F: int,
                   token_mask: Optional[np.ndarray] = None, nthreads: int = 0,
                   eps: float = STACK_EPS) -> ChainResult:
    """L MoE layers in sequence on one residual stream (the resident engine
    running the model layer after layer, [P3-PK] / [P5-TRT]).  Reading: the
    pages describe the MoE layer alone; between two of them the stream is a
    pre-norm residual block without its attention, whose normalisation (one
    of the per-operator model's operators, [P3-PK]) has unit gain, as the
    synthetic model has no trained norm weights:
      r_0 = x;  x_l = bf16(r_l / sqrt(mean(r_l^2) + eps));
      r_{l+1} = r_l + MoE_l(x_l);  result r_L.
    (Without the normalisation the stream grows layer over layer: SwiGLU is
    quadratic in its input, and eight layers of these weights overflow fp32.)
    The rounding to bf16 decides the next layer's input, so it is taken in the
    kernel's precision: to the nearest fp32, then to the nearest bf16
    (round_bf16).  Sums and the normalisation are fp64.  token_mask: every
    layer computes all routing but only the masked tokens' expert pairs, and
    the unmasked tokens' later inputs are then not computed (so the mask is
    for T = 1 stacks or for timing only)."""
    L = len(w_r)
    assert len(packed) == L and len(scales) == L
    x0 = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    r = (x0.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    res, xs = [], []
    for l in range(L):
        x = round_bf16(rms_normalize(r, eps))
        xs.append(x)
        o = forward(x, w_r[l], packed[l], scales[l], k, F, token_mask=token_mask, nthreads=nthreads)
        res.append(o)
        r = r + o.out
    return ChainResult(r, res, xs, float(min(o.min_gap for o in res)))
