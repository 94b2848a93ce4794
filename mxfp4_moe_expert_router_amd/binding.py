"""ctypes binding of libmoe_mxfp4.so (the C ABI in include/moe_mxfp4.h).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  PyTorch provides the device memory (tensors) and the stream.  If the
library has not been built, importing this module raises: there is no other
code path.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe_mxfp4.so")

MOE_OK, MOE_EINVAL, MOE_ESHAPE, MOE_EWORKSPACE, MOE_ELAUNCH, MOE_ETIMEOUT, MOE_EDEVICE, MOE_EALIGN = range(8)
MOE_OPT_WITHHOLD_ARRIVAL = 0x1
MOE_OPT_TRACE = 0x2
MOE_OPT_COOPERATIVE = 0x4
MOE_OPT_WITHHOLD_H = 0x8
MOE_QDTYPE_F32, MOE_QDTYPE_BF16 = 0, 1
MOE_LAYERS_PER_LAUNCH = 0x1
MOE_LAYERS_ONE_LAUNCH = 0x2
MOE_LAYERS_COOPERATIVE = 0x4


class MoeError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        super().__init__(f"{what}: {strerror(status)} ({status})" if what else f"{strerror(status)} ({status})")


class Dims(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("d", ctypes.c_int32), ("ffn", ctypes.c_int32), ("E", ctypes.c_int32)]


class Options(ctypes.Structure):
    _fields_ = [("flags", ctypes.c_uint32), ("spin_limit_us", ctypes.c_uint32), ("grid", ctypes.c_int32)]


class WsLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in
                ("logits", "topk_idx", "topk_w", "offsets", "sorted_slot", "pos", "active", "n_active", "h", "y", "trace",
                 "x_last", "h_chunk_major", "total")]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"HIP library not built: {LIB_PATH} is missing "
                          f"(run python mxfp4_moe_expert_router_amd/build.py)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    P = ctypes.POINTER
    lib.moe_mxfp4_expert_packed_bytes.restype = sz
    lib.moe_mxfp4_expert_packed_bytes.argtypes = [i32, i32]
    lib.moe_mxfp4_expert_scale_bytes.restype = sz
    lib.moe_mxfp4_expert_scale_bytes.argtypes = [i32, i32]
    lib.moe_mxfp4_workspace_bytes.restype = sz
    lib.moe_mxfp4_workspace_bytes.argtypes = [P(Dims), i32]
    lib.moe_mxfp4_workspace_init.restype = ctypes.c_int
    lib.moe_mxfp4_workspace_init.argtypes = [vp, sz, vp]
    fwd = [P(Dims), vp, vp, vp, vp, i32, vp, vp, sz]
    lib.moe_mxfp4_forward.restype = ctypes.c_int
    lib.moe_mxfp4_forward.argtypes = fwd + [vp]
    lib.moe_mxfp4_forward_staged.restype = ctypes.c_int
    lib.moe_mxfp4_forward_staged.argtypes = fwd + [vp]
    lib.moe_mxfp4_forward_noalloc.restype = ctypes.c_int
    lib.moe_mxfp4_forward_noalloc.argtypes = [P(Dims), vp, vp, vp, vp, i32, vp, vp]
    lib.moe_mxfp4_forward_ex.restype = ctypes.c_int
    lib.moe_mxfp4_forward_ex.argtypes = fwd + [P(Options), vp]
    lib.moe_mxfp4_route.restype = ctypes.c_int
    lib.moe_mxfp4_route.argtypes = [P(Dims), vp, vp, i32, vp, vp, vp, vp, vp, sz, vp]
    lib.moe_mxfp4_workspace_layout.restype = ctypes.c_int
    lib.moe_mxfp4_workspace_layout.argtypes = [P(Dims), i32, P(WsLayout)]
    lib.moe_mxfp4_status.restype = ctypes.c_int
    lib.moe_mxfp4_status.argtypes = [vp, vp]
    lib.moe_mxfp4_strerror.restype = ctypes.c_char_p
    lib.moe_mxfp4_strerror.argtypes = [ctypes.c_int]
    lib.moe_mxfp4_persistent_grid.restype = ctypes.c_int
    lib.moe_mxfp4_persistent_grid.argtypes = [P(Dims), i32]
    lib.moe_mxfp4_quantize.restype = ctypes.c_int
    lib.moe_mxfp4_forward_layers.restype = ctypes.c_int
    lib.moe_mxfp4_forward_layers.argtypes = [P(Dims), i32, vp, vp, vp, vp, i32, vp, vp, sz, i32, vp]
    lib.moe_mxfp4_layers_one_launch.restype = ctypes.c_int
    lib.moe_mxfp4_layers_one_launch.argtypes = [P(Dims), i32]
    lib.moe_mxfp4_quantize.argtypes = [vp, i32, ctypes.c_int64, ctypes.c_int64, vp, vp, vp]
    lib.moe_mxfp4_quantize_host.restype = ctypes.c_int
    lib.moe_mxfp4_quantize_host.argtypes = [vp, ctypes.c_int64, ctypes.c_int64, vp, vp]
    lib.moe_mxfp4_dequantize_host.restype = ctypes.c_int
    lib.moe_mxfp4_dequantize_host.argtypes = [vp, vp, ctypes.c_int64, ctypes.c_int64, vp]
    return lib


lib = _load()


def strerror(status: int) -> str:
    return lib.moe_mxfp4_strerror(status).decode()


def _check(st: int, what: str):
    if st != MOE_OK:
        raise MoeError(st, what)


def _stream(stream=None) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


@dataclass(frozen=True)
class LayerDims:
    T: int
    d: int
    ffn: int
    E: int

    def c(self) -> Dims:
        return Dims(self.T, self.d, self.ffn, self.E)


def expert_packed_bytes(d: int, ffn: int) -> int:
    return int(lib.moe_mxfp4_expert_packed_bytes(d, ffn))


def expert_scale_bytes(d: int, ffn: int) -> int:
    return int(lib.moe_mxfp4_expert_scale_bytes(d, ffn))


def workspace_bytes(dims: LayerDims, topk: int) -> int:
    n = int(lib.moe_mxfp4_workspace_bytes(ctypes.byref(dims.c()), topk))
    if n == 0:
        raise MoeError(MOE_ESHAPE, "workspace_bytes")
    return n


def alloc_workspace(dims: LayerDims, topk: int, device="cuda") -> torch.Tensor:
    """Zero-filled workspace (required before its first use)."""
    return torch.zeros(workspace_bytes(dims, topk), dtype=torch.uint8, device=device)


def workspace_layout(dims: LayerDims, topk: int) -> WsLayout:
    lay = WsLayout()
    _check(lib.moe_mxfp4_workspace_layout(ctypes.byref(dims.c()), topk, ctypes.byref(lay)), "workspace_layout")
    return lay


def persistent_grid(dims: LayerDims, topk: int) -> int:
    g = lib.moe_mxfp4_persistent_grid(ctypes.byref(dims.c()), topk)
    if g < 0:
        raise MoeError(-g, "persistent_grid")
    return g


def dims_of(x: torch.Tensor, router_w: torch.Tensor, packed: torch.Tensor) -> LayerDims:
    T, d = x.shape
    E = router_w.shape[0]
    ffn = packed.shape[-1] * 2 // (3 * d) if packed.dim() == 2 else packed.numel() * 2 // (3 * d * E)
    return LayerDims(int(T), int(d), int(ffn), int(E))


def _validate(x, router_w, packed, scales, out, dims: Optional[LayerDims] = None, layers: int = 1):
    """dtype, contiguity and (with dims) element counts of every tensor given,
    then that each lives on the device: a short buffer would otherwise let a
    kernel read or write past its end."""
    want = {}
    if dims is not None:
        T, d, F, E = dims.T, dims.d, dims.ffn, dims.E
        want = {"x": T * d, "router_w": layers * E * d, "packed": layers * E * 3 * d * F // 2,
                "scales": layers * E * 3 * d * F // 32, "out": T * d}
    named = (("x", x, torch.bfloat16), ("router_w", router_w, torch.float32), ("packed", packed, torch.uint8),
             ("scales", scales, torch.uint8), ("out", out, torch.float32))
    for name, t, dt in named:
        if t is None:
            continue
        if t.dtype != dt and not (name == "x" and t.dtype == torch.int16):
            raise ValueError(f"{name} must be {dt}, got {t.dtype}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if name in want and t.numel() != want[name]:
            raise ValueError(f"{name} has {t.numel()} elements, the sizes need {want[name]}")
    for name, t, _ in named:
        if t is not None and not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")


def forward(x: torch.Tensor, router_w: torch.Tensor, packed: torch.Tensor, scales: torch.Tensor, topk: int,
            out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None, staged: bool = False,
            options: Optional[Options] = None, stream=None, dims: Optional[LayerDims] = None) -> torch.Tensor:
    """One MoE layer.  x bf16 [T, d]; router_w fp32 [E, d]; packed uint8 [E, 3*d*ffn/2];
    scales uint8 [E, 3*d*ffn/32]; returns out fp32 [T, d]."""
    dims = dims or dims_of(x, router_w, packed)
    if out is None:
        out = torch.empty((dims.T, dims.d), dtype=torch.float32, device=x.device)
    _validate(x, router_w, packed, scales, out, dims)
    if workspace is None:
        workspace = alloc_workspace(dims, topk, x.device)
    cd = dims.c()
    args = (ctypes.byref(cd), _ptr(x), _ptr(router_w), _ptr(packed), _ptr(scales), int(topk), _ptr(out),
            _ptr(workspace), workspace.numel())
    if staged:
        st = lib.moe_mxfp4_forward_staged(*args, _stream(stream))
    elif options is not None:
        st = lib.moe_mxfp4_forward_ex(*args, ctypes.byref(options), _stream(stream))
    else:
        st = lib.moe_mxfp4_forward(*args, _stream(stream))
    _check(st, "moe_mxfp4_forward" + ("_staged" if staged else ""))
    return out


def forward_noalloc(x: torch.Tensor, router_w: torch.Tensor, packed: torch.Tensor, scales: torch.Tensor,
                    topk: int, out: torch.Tensor, stream=None, dims: Optional[LayerDims] = None) -> torch.Tensor:
    """One MoE layer on the library's own device workspace
    (moe_mxfp4_forward_noalloc): nothing is allocated; `out` fp32 [T, d] is
    the caller's."""
    dims = dims or dims_of(x, router_w, packed)
    _validate(x, router_w, packed, scales, out, dims)
    st = lib.moe_mxfp4_forward_noalloc(ctypes.byref(dims.c()), _ptr(x), _ptr(router_w), _ptr(packed), _ptr(scales),
                                       int(topk), _ptr(out), _stream(stream))
    _check(st, "moe_mxfp4_forward_noalloc")
    return out


def forward_raw(dims: LayerDims, x_ptr: int, wr_ptr: int, packed_ptr: int, scales_ptr: int, topk: int, out_ptr: int,
                ws_ptr: int, ws_bytes: int, stream_handle: int, staged: bool = False) -> int:
    """Unchecked pointer-level call (bench loops); returns the status."""
    fn = lib.moe_mxfp4_forward_staged if staged else lib.moe_mxfp4_forward
    return fn(ctypes.byref(dims.c()), x_ptr, wr_ptr, packed_ptr, scales_ptr, topk, out_ptr, ws_ptr, ws_bytes,
              stream_handle)


def forward_layers(x: torch.Tensor, router_w: torch.Tensor, packed: torch.Tensor, scales: torch.Tensor, topk: int,
                   out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None, flags: int = 0,
                   stream=None, dims: Optional[LayerDims] = None) -> torch.Tensor:
    """A stack of L MoE layers on one residual stream, each on the unit-gain RMS
    normalised stream (moe_mxfp4_forward_layers):
    x bf16 [T, d]; router_w fp32 [L, E, d]; packed uint8 [L, E, 3*d*ffn/2];
    scales uint8 [L, E, 3*d*ffn/32]; returns out fp32 [T, d] = r_L."""
    if router_w.dim() != 3 or packed.dim() != 3 or scales.dim() != 3:
        raise ValueError("router_w, packed and scales must be [L, E, ...]")
    L, E, d = router_w.shape
    if packed.shape[:2] != (L, E) or scales.shape[:2] != (L, E):
        raise ValueError("router_w, packed and scales disagree on L or E")
    dims = dims or LayerDims(int(x.shape[0]), int(d), int(packed.shape[2] * 2 // (3 * d)), int(E))
    if out is None:
        out = torch.empty((dims.T, dims.d), dtype=torch.float32, device=x.device)
    _validate(x, router_w, packed, scales, out, dims, int(L))
    if workspace is None:
        workspace = alloc_workspace(dims, topk, x.device)
    st = lib.moe_mxfp4_forward_layers(ctypes.byref(dims.c()), int(L), _ptr(x), _ptr(router_w), _ptr(packed),
                                      _ptr(scales), int(topk), _ptr(out), _ptr(workspace), workspace.numel(),
                                      int(flags), _stream(stream))
    _check(st, "moe_mxfp4_forward_layers")
    return out


def forward_layers_raw(dims: LayerDims, layers: int, x_ptr: int, wr_ptr: int, packed_ptr: int, scales_ptr: int,
                       topk: int, out_ptr: int, ws_ptr: int, ws_bytes: int, flags: int, stream_handle: int) -> int:
    """Unchecked pointer-level stack call (bench loops); returns the status."""
    return lib.moe_mxfp4_forward_layers(ctypes.byref(dims.c()), layers, x_ptr, wr_ptr, packed_ptr, scales_ptr, topk,
                                        out_ptr, ws_ptr, ws_bytes, flags, stream_handle)


def layers_one_launch(dims: LayerDims, topk: int) -> bool:
    """True if forward_layers can run these sizes as one resident launch (MOE_LAYERS_ONE_LAUNCH)."""
    r = lib.moe_mxfp4_layers_one_launch(ctypes.byref(dims.c()), topk)
    if r < 0:
        raise MoeError(-r, "layers_one_launch")
    return bool(r)


def route(x: torch.Tensor, router_w: torch.Tensor, topk: int, ffn: int, workspace: Optional[torch.Tensor] = None,
          stream=None):
    """Routing only: (topk_idx int32 [T,k], topk_w fp32 [T,k], offsets int32 [E+1], sorted_slot int32 [T*k])."""
    T, d = x.shape
    E = router_w.shape[0]
    dims = LayerDims(int(T), int(d), int(ffn), int(E))
    _validate(x, router_w, None, None, None, dims)
    if workspace is None:
        workspace = alloc_workspace(dims, topk, x.device)
    dev = x.device
    idx = torch.empty((T, topk), dtype=torch.int32, device=dev)
    w = torch.empty((T, topk), dtype=torch.float32, device=dev)
    off = torch.empty(E + 1, dtype=torch.int32, device=dev)
    ss = torch.empty(T * topk, dtype=torch.int32, device=dev)
    cd = dims.c()
    st = lib.moe_mxfp4_route(ctypes.byref(cd), _ptr(x), _ptr(router_w), int(topk), _ptr(idx), _ptr(w), _ptr(off),
                             _ptr(ss), _ptr(workspace), workspace.numel(), _stream(stream))
    _check(st, "moe_mxfp4_route")
    return idx, w, off, ss


def status(workspace: torch.Tensor, stream=None) -> int:
    return int(lib.moe_mxfp4_status(_ptr(workspace), _stream(stream)))


def workspace_init(workspace: torch.Tensor, stream=None):
    _check(lib.moe_mxfp4_workspace_init(_ptr(workspace), workspace.numel(), _stream(stream)), "workspace_init")


def intermediates(workspace: torch.Tensor, dims: LayerDims, topk: int) -> dict:
    """Views of the intermediates a forward call left in `workspace`."""
    lay = workspace_layout(dims, topk)
    T, E, F, d, TK = dims.T, dims.E, dims.ffn, dims.d, dims.T * topk

    def view(off, n, dt):
        nbytes = n * torch.tensor([], dtype=dt).element_size()
        return workspace[off: off + nbytes].view(dt)

    def tagged(off, n):
        words = workspace[off: off + n * 8].view(torch.int32).view(n, 2)
        return words[:, 0].contiguous().view(torch.float32)

    h = tagged(lay.h, TK * F).view(TK, F)
    if lay.h_chunk_major:  # row order: value 32 c + e at word 2 ((e / 2) (F / 32) + c) + e % 2
        h = h.view(TK, 16, F // 32, 2).permute(0, 2, 1, 3).reshape(TK, F)
    return {
        "logits": view(lay.logits, T * E, torch.float32).view(T, E),
        "topk_idx": view(lay.topk_idx, TK, torch.int32).view(T, topk),
        "topk_w": view(lay.topk_w, TK, torch.float32).view(T, topk),
        "offsets": view(lay.offsets, E + 1, torch.int32),
        "sorted_slot": view(lay.sorted_slot, TK, torch.int32),
        "pos": view(lay.pos, TK, torch.int32),
        "active": view(lay.active, E, torch.int32),
        "n_active": view(lay.n_active, 1, torch.int32),
        "h": h,
        "y": tagged(lay.y, TK * d).view(TK, d),
        "trace": view(lay.trace, 2048 * 16, torch.int64).view(2048, 16),
        "x_last": view(lay.x_last, T * d, torch.int16).view(T, d),
    }


def quantize(w: torch.Tensor, packed: Optional[torch.Tensor] = None, scales: Optional[torch.Tensor] = None,
             stream=None):
    """MXFP4 quantize/pack of a 2-D fp32 or bf16 device tensor [rows, K] on the GPU
    (moe_mxfp4_quantize): returns (packed uint8 [rows, K/2], scales uint8 [rows, K/32])."""
    if w.dim() != 2 or w.dtype not in (torch.float32, torch.bfloat16) or not w.is_contiguous():
        raise ValueError("w must be a contiguous 2-D fp32 or bf16 tensor")
    rows, K = w.shape
    if packed is None:
        packed = torch.empty((rows, K // 2), dtype=torch.uint8, device=w.device)
    if scales is None:
        scales = torch.empty((rows, K // 32), dtype=torch.uint8, device=w.device)
    for name, t, n in (("packed", packed, rows * (K // 2)), ("scales", scales, rows * (K // 32))):
        if t.dtype != torch.uint8 or not t.is_contiguous() or t.numel() != n:
            raise ValueError(f"{name} must be a contiguous uint8 tensor of {n} elements")
    if not (w.is_cuda and packed.is_cuda and scales.is_cuda):
        raise ValueError("w, packed and scales must be device tensors")
    dt = MOE_QDTYPE_F32 if w.dtype == torch.float32 else MOE_QDTYPE_BF16
    _check(lib.moe_mxfp4_quantize(_ptr(w), dt, rows, K, _ptr(packed), _ptr(scales), _stream(stream)), "quantize")
    return packed, scales


def quantize_host(w):
    """MXFP4 quantize/pack of a 2-D fp32 host array [rows, K] in the library's
    host code (moe_mxfp4_quantize_host): returns (packed uint8 [rows, K/2],
    scales uint8 [rows, K/32]) as numpy arrays."""
    import numpy as np

    w = np.ascontiguousarray(w, dtype=np.float32)
    if w.ndim != 2:
        raise ValueError("w must be 2-D")
    rows, K = w.shape
    packed = np.zeros((rows, K // 2), dtype=np.uint8)
    scales = np.zeros((rows, K // 32), dtype=np.uint8)
    _check(lib.moe_mxfp4_quantize_host(w.ctypes.data, rows, K, packed.ctypes.data, scales.ctypes.data),
           "quantize_host")
    return packed, scales


def dequantize_host(packed, scales, rows: int, K: int):
    """MXFP4 codes and scales (host arrays) -> fp32 [rows, K]
    (moe_mxfp4_dequantize_host)."""
    import numpy as np

    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    if packed.size != rows * (K // 2) or scales.size != rows * (K // 32):
        raise ValueError("packed / scales sizes do not match rows and K")
    w = np.empty((rows, K), dtype=np.float32)
    _check(lib.moe_mxfp4_dequantize_host(packed.ctypes.data, scales.ctypes.data, rows, K, w.ctypes.data),
           "dequantize_host")
    return w
