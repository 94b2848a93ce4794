"""Seeded synthetic inputs shared by the GPU library's tests/bench and the CPU oracle.

The input recipe of the layer's workloads (bf16 activations ~N(0,1), fp32
router weights ~N(0,0.05), expert gate/up/down weights ~N(0,0.02) stored as
MXFP4), plus the Zipf(s) expert-popularity bias of the batched-verify
workload.  Nothing here routes, decodes or computes the layer; see gen.c for
the generator and the storage format it writes.

Seeds: every workload has a base seed (0).  Expert weights always come from
the base seed, so all full-size workloads share one set of expert weights.
Activations and router weights come from a "route seed", the first seed at or
after the base whose every token has a gap larger than 1e-3 between its k-th
and (k+1)-th router logit; tests/golden/make_seeds.py finds it with the
oracle and records it (with the Zipf strength) in tests/golden/seeds.json.
"""
from __future__ import annotations

import ctypes
import json
import math
import os
import subprocess
from dataclasses import dataclass, replace
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_SEEDS_PATH = os.path.join(os.path.dirname(_HERE), "tests", "golden", "seeds.json")

# Stream ids of the tensors (see gen.c: synth_stream_key).
TENSOR_X, TENSOR_WR, TENSOR_ZIPF, TENSOR_XSHARED = 0, 1, 5, 6


@dataclass(frozen=True)
class Config:
    """One workload: T tokens, hidden d, expert ffn F, E experts, top-k."""

    name: str
    T: int
    d: int
    F: int
    E: int
    k: int
    zipf_s: Optional[float] = None  # Zipf exponent of expert popularity, None = unbiased
    zipf_beta: float = 0.0  # logit bias strength: b_e = -beta * s * ln(rank_e)
    x_shared: float = 0.0  # share of each token's variance in a component common to all tokens
    seed: int = 0  # base seed (expert weights)
    route_seed: int = 0  # seed of activations / router weights
    x_std: float = 1.0
    wr_std: float = 0.05
    w_std: float = 0.02

    def with_T(self, T: int) -> "Config":
        return replace(self, T=T, name=f"{self.name}_T{T}")


# The five workloads of the layer, and the verify-block sizes of the sweep.
_BASE = {
    "tiny": Config("tiny", T=8, d=256, F=128, E=8, k=2),
    "decode": Config("decode", T=1, d=7168, F=2048, E=256, k=8),
    "verify": Config("verify", T=8, d=7168, F=2048, E=256, k=8),
    "batched_verify": Config("batched_verify", T=128, d=7168, F=2048, E=256, k=8, zipf_s=1.1),
    "dense": Config("dense", T=512, d=7168, F=2048, E=256, k=8),
    # verify-block size sweep (uniform routing, same shapes as verify)
    "sweep_T4": Config("sweep_T4", T=4, d=7168, F=2048, E=256, k=8),
    "sweep_T16": Config("sweep_T16", T=16, d=7168, F=2048, E=256, k=8),
    "sweep_T22": Config("sweep_T22", T=22, d=7168, F=2048, E=256, k=8),
    "sweep_T32": Config("sweep_T32", T=32, d=7168, F=2048, E=256, k=8),
    # a verify block of consecutive positions: the tokens share 70% of their
    # variance, so they overlap in their experts (30 active, up to 7 tokens)
    "verify_shared": Config("verify_shared", T=8, d=7168, F=2048, E=256, k=8, x_shared=0.7),
}


def _load_seeds() -> dict:
    if os.path.exists(_SEEDS_PATH):
        with open(_SEEDS_PATH) as f:
            return json.load(f)
    return {}


def get_config(name: str) -> Config:
    cfg = _BASE[name]
    rec = _load_seeds().get(name)
    if rec:
        cfg = replace(cfg, route_seed=int(rec["route_seed"]), zipf_beta=float(rec.get("zipf_beta", 0.0)))
    return cfg


def config_names():
    return list(_BASE)


# ----------------------------------------------------------------------------- native generator


def build(force: bool = False) -> str:
    """Compile gen.c into libsynth.so next to it (gcc, OpenMP)."""
    src = os.path.join(_HERE, "gen.c")
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(src):
        tmp = _LIB_PATH + f".tmp{os.getpid()}"
        subprocess.run(
            ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", src, "-o", tmp, "-lm"],
            check=True,
        )
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def _L():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        u64, u32, i64, i32 = ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int64, ctypes.c_int
        vp = ctypes.c_void_p
        lib.synth_stream_key.restype = u64
        lib.synth_stream_key.argtypes = [u64, u32, u32]
        lib.synth_u64.restype = u64
        lib.synth_u64.argtypes = [u64, u64]
        lib.synth_normal_f32.restype = None
        lib.synth_normal_f32.argtypes = [u64, u64, i64, ctypes.c_float, vp]
        lib.synth_f32_to_bf16.restype = None
        lib.synth_f32_to_bf16.argtypes = [vp, i64, vp]
        lib.synth_quantize_mxfp4.restype = None
        lib.synth_quantize_mxfp4.argtypes = [vp, i64, i64, vp, vp]
        lib.synth_experts.restype = i32
        lib.synth_experts.argtypes = [u64, i32, i32, i32, i32, ctypes.c_float, vp, vp, i32]
        _lib = lib
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def stream_key(seed: int, tensor: int, index: int) -> int:
    return int(_L().synth_stream_key(seed, tensor, index))


def normals(seed: int, tensor: int, index: int, n: int, std: float, start: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    _L().synth_normal_f32(stream_key(seed, tensor, index), start, n, std, _ptr(out))
    return out


def f32_to_bf16(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.uint16)
    _L().synth_f32_to_bf16(_ptr(a), a.size, _ptr(out))
    return out


def bf16_to_f32(u: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp32 (exact)."""
    return (np.asarray(u, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def quantize_mxfp4(w: np.ndarray):
    """Pack fp32 rows [rows, K] into (packed uint8 [rows, K/2], scales uint8 [rows, K/32])."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    rows, K = w.shape
    assert K % 32 == 0
    packed = np.empty((rows, K // 2), dtype=np.uint8)
    scales = np.empty((rows, K // 32), dtype=np.uint8)
    _L().synth_quantize_mxfp4(_ptr(w), rows, K, _ptr(packed), _ptr(scales))
    return packed, scales


# ----------------------------------------------------------------------------- workload inputs


def expert_packed_bytes(d: int, F: int) -> int:
    return 3 * d * F // 2


def expert_scale_bytes(d: int, F: int) -> int:
    return 3 * d * F // 32


def zipf_ranks(cfg: Config) -> np.ndarray:
    """rank_e in 1..E: a seeded random permutation of experts (Fisher-Yates)."""
    key = stream_key(cfg.route_seed, TENSOR_ZIPF, 0)
    perm = np.arange(cfg.E)
    for i in range(cfg.E - 1, 0, -1):
        j = int(_L().synth_u64(key, i)) % (i + 1)
        perm[i], perm[j] = perm[j], perm[i]
    ranks = np.empty(cfg.E, dtype=np.int64)
    ranks[perm] = np.arange(1, cfg.E + 1)
    return ranks


def zipf_bias(cfg: Config, beta: Optional[float] = None) -> np.ndarray:
    """Logit bias b_e = -beta * s * ln(rank_e) (popularity p_e ~ rank_e^-s)."""
    beta = cfg.zipf_beta if beta is None else beta
    r = zipf_ranks(cfg).astype(np.float64)
    return (-beta * cfg.zipf_s * np.log(r)).astype(np.float32)


def routing_inputs(cfg: Config, beta: Optional[float] = None):
    """(x bf16 bits uint16 [T, d], router weights fp32 [E, d]).

    With x_shared = s > 0, every token is sqrt(s) c + sqrt(1 - s) n_t with one
    common normal vector c (stream TENSOR_XSHARED) and its own n_t.
    With a Zipf workload, column 0 carries the popularity bias: x[:, 0] = 1
    and W_r[:, 0] = b_e, so every token's logit for expert e gains b_e.
    """
    x32 = normals(cfg.route_seed, TENSOR_X, 0, cfg.T * cfg.d, cfg.x_std).reshape(cfg.T, cfg.d)
    if cfg.x_shared > 0:
        # x_t = sqrt(s) c + sqrt(1 - s) n_t: common c, own n_t, same variance
        c = normals(cfg.route_seed, TENSOR_XSHARED, 0, cfg.d, cfg.x_std)
        x32 = (np.float32(math.sqrt(cfg.x_shared)) * c[None, :]
               + np.float32(math.sqrt(1.0 - cfg.x_shared)) * x32).astype(np.float32)
    wr = normals(cfg.route_seed, TENSOR_WR, 0, cfg.E * cfg.d, cfg.wr_std).reshape(cfg.E, cfg.d)
    if cfg.zipf_s is not None:
        x32[:, 0] = 1.0
        wr[:, 0] = zipf_bias(cfg, beta)
    return f32_to_bf16(x32), np.ascontiguousarray(wr)


def expert_weights(cfg: Config, out_packed: Optional[np.ndarray] = None,
                   out_scales: Optional[np.ndarray] = None, e0: int = 0, e1: Optional[int] = None,
                   nthreads: int = 0):
    """Packed experts [e1-e0, 3dF/2] and their scales [e1-e0, 3dF/32] (uint8)."""
    e1 = cfg.E if e1 is None else e1
    n = e1 - e0
    pb, sb = expert_packed_bytes(cfg.d, cfg.F), expert_scale_bytes(cfg.d, cfg.F)
    packed = np.empty((n, pb), dtype=np.uint8) if out_packed is None else out_packed
    scales = np.empty((n, sb), dtype=np.uint8) if out_scales is None else out_scales
    assert packed.shape == (n, pb) and scales.shape == (n, sb)
    if nthreads <= 0:
        nthreads = min(16, os.cpu_count() or 1)
    rc = _L().synth_experts(cfg.seed, e0, e1, cfg.d, cfg.F, cfg.w_std, _ptr(packed), _ptr(scales), nthreads)
    if rc != 0:
        raise RuntimeError(f"synth_experts failed ({rc})")
    return packed, scales


def chain_layer_config(cfg: Config, layer: int) -> Config:
    """Inputs of layer `layer` of a stack of MoE layers on one residual stream:
    layer 0 is `cfg` itself; layer l draws its expert weights from seed
    cfg.seed + l and its router weights from route seed cfg.route_seed + l
    (its activations come from the layer before, not from this seed)."""
    if layer == 0:
        return cfg
    return replace(cfg, name=f"{cfg.name}_layer{layer}", seed=cfg.seed + layer, route_seed=cfg.route_seed + layer)


def algorithmic_bytes(cfg: Config, n_active: int) -> int:
    """Bytes the layer must move: each active expert's packed+scale bytes once,
    the router weights, the activations and the fp32 output."""
    per_expert = expert_packed_bytes(cfg.d, cfg.F) + expert_scale_bytes(cfg.d, cfg.F)
    return n_active * per_expert + cfg.E * cfg.d * 4 + cfg.T * cfg.d * 2 + cfg.T * cfg.d * 4


def layer_flops(cfg: Config) -> int:
    """2*(3*d*F) per (token, expert) pair plus 2*T*E*d for the router."""
    return 2 * 3 * cfg.d * cfg.F * cfg.T * cfg.k + 2 * cfg.T * cfg.E * cfg.d


__all__ = [
    "Config", "get_config", "config_names", "build", "routing_inputs", "expert_weights", "chain_layer_config",
    "quantize_mxfp4", "f32_to_bf16", "bf16_to_f32", "normals", "zipf_ranks", "zipf_bias",
    "expert_packed_bytes", "expert_scale_bytes", "algorithmic_bytes", "layer_flops", "math",
]
