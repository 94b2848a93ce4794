"""The C-ABI library without a GPU: it loads, exports every function that
include/moe_mxfp4.h declares, and rejects bad arguments with the documented
status codes before enqueuing anything."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_mxfp4.h")


@pytest.fixture(scope="module")
def moe():
    import mxfp4_moe_expert_router_amd as m
    return m


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_mxfp4_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol(moe):
    names = declared_functions()
    assert len(names) >= 12
    lib = ctypes.CDLL(moe.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in include/moe_mxfp4.h but not exported"


def test_sizes(moe):
    assert moe.expert_packed_bytes(7168, 2048) == 3 * 7168 * 2048 // 2 == 22020096
    assert moe.expert_scale_bytes(7168, 2048) == 3 * 7168 * 2048 // 32 == 1376256
    d = moe.LayerDims(8, 7168, 2048, 256)
    ws = moe.workspace_bytes(d, 8)
    lay = moe.workspace_layout(d, 8)
    assert lay.total == ws
    assert lay.h % 256 == 0 and lay.y % 256 == 0
    assert lay.y - lay.h >= 64 * 2048 * 4 and ws - lay.y >= 64 * 7168 * 4


def _call(moe, dims, topk=2, x=256, wr=256, p=256, s=256, out=256, ws=256, wsb=1 << 30):
    D = moe.binding.Dims(*dims)
    return moe.binding.lib.moe_mxfp4_forward(ctypes.byref(D), x, wr, p, s, topk, out, ws, wsb, None)


def test_validation_codes(moe):
    ok_dims = (4, 64, 32, 8)
    assert _call(moe, ok_dims, x=0) == moe.MOE_EINVAL
    assert _call(moe, ok_dims, ws=0) == moe.MOE_EINVAL
    assert _call(moe, ok_dims, topk=0) == moe.MOE_EINVAL
    assert _call(moe, ok_dims, topk=9) == moe.MOE_EINVAL
    assert _call(moe, (-1, 64, 32, 8)) == moe.MOE_EINVAL
    assert _call(moe, (4, 48, 32, 8)) == moe.MOE_ESHAPE
    assert _call(moe, (4, 64, 40, 8)) == moe.MOE_ESHAPE
    assert _call(moe, (4, 64, 32, 2048), topk=2) == moe.MOE_ESHAPE
    assert _call(moe, (4096, 64, 32, 256)) == moe.MOE_ESHAPE  # permutation mask limit
    assert _call(moe, ok_dims, x=264) == moe.MOE_EALIGN
    assert _call(moe, ok_dims, ws=512 + 16) == moe.MOE_EALIGN
    assert _call(moe, ok_dims, wsb=1024) == moe.MOE_EWORKSPACE
    assert _call(moe, (0, 64, 32, 8)) == moe.MOE_OK  # empty batch: nothing to do
    assert _call(moe, (0, 64, 32, 8), x=0, out=0) == moe.MOE_OK  # empty tensors may be null
    assert moe.workspace_bytes(moe.LayerDims(4, 64, 32, 8), 2) > 0
    with pytest.raises(moe.MoeError):
        moe.workspace_bytes(moe.LayerDims(4, 48, 32, 8), 2)


def test_strerror(moe):
    for st in range(8):
        assert moe.strerror(st)
    assert moe.strerror(99) == "unknown status"


def test_quantize_rejects_bad_arguments(moe):
    """moe_mxfp4_quantize validates on the host before touching the device."""
    lib = ctypes.CDLL(moe.LIB_PATH)
    q = lib.moe_mxfp4_quantize
    q.restype = ctypes.c_int
    q.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                  ctypes.c_void_p]
    assert q(None, moe.MOE_QDTYPE_F32, 0, 64, None, None, None) == moe.MOE_OK  # nothing to do
    assert q(None, moe.MOE_QDTYPE_F32, 4, 0, None, None, None) == moe.MOE_OK
    assert q(None, moe.MOE_QDTYPE_F32, 4, 48, None, None, None) == moe.MOE_ESHAPE  # K % 32
    assert q(None, 7, 4, 64, None, None, None) == moe.MOE_EINVAL  # dtype
    assert q(None, moe.MOE_QDTYPE_BF16, -1, 64, None, None, None) == moe.MOE_EINVAL
    assert q(None, moe.MOE_QDTYPE_F32, 4, 64, None, None, None) == moe.MOE_EINVAL  # null pointers
    buf = ctypes.create_string_buffer(64 * 4 * 4 + 32)
    base = (ctypes.addressof(buf) + 15) // 16 * 16
    assert q(base + 4, moe.MOE_QDTYPE_F32, 4, 64, base, base, None) == moe.MOE_EALIGN


def _call_layers(moe, dims, layers=2, topk=2, flags=0, x=256, wr=256, p=256, s=256, out=256, ws=256, wsb=1 << 30):
    D = moe.binding.Dims(*dims)
    return moe.binding.lib.moe_mxfp4_forward_layers(ctypes.byref(D), layers, x, wr, p, s, topk, out, ws, wsb, flags,
                                                    None)


def test_layers_validation_codes(moe):
    ok_dims = (4, 64, 32, 8)
    assert _call_layers(moe, ok_dims, layers=0) == moe.MOE_EINVAL
    assert _call_layers(moe, ok_dims, layers=4097) == moe.MOE_EINVAL
    assert _call_layers(moe, ok_dims, flags=8) == moe.MOE_EINVAL
    assert _call_layers(moe, ok_dims, flags=moe.MOE_LAYERS_PER_LAUNCH | moe.MOE_LAYERS_ONE_LAUNCH) == moe.MOE_EINVAL
    assert _call_layers(moe, ok_dims, x=0) == moe.MOE_EINVAL
    assert _call_layers(moe, ok_dims, topk=9) == moe.MOE_EINVAL
    assert _call_layers(moe, (4, 48, 32, 8)) == moe.MOE_ESHAPE
    assert _call_layers(moe, ok_dims, out=264) == moe.MOE_EALIGN
    assert _call_layers(moe, ok_dims, wsb=1024) == moe.MOE_EWORKSPACE
    assert _call_layers(moe, (0, 64, 32, 8), x=0, out=0) == moe.MOE_OK
    # the dense batch takes the MFMA path: one launch per layer only
    assert _call_layers(moe, (512, 7168, 2048, 256), topk=8, flags=moe.MOE_LAYERS_ONE_LAUNCH) == moe.MOE_ESHAPE


def test_layers_one_launch_choice(moe):
    assert moe.layers_one_launch(moe.LayerDims(8, 7168, 2048, 256), 8)      # verify block: x of all tokens in LDS
    assert moe.layers_one_launch(moe.LayerDims(1, 7168, 2048, 256), 8)      # decode
    assert not moe.layers_one_launch(moe.LayerDims(32, 7168, 2048, 256), 8)  # x rows of the workgroup's pairs
    assert not moe.layers_one_launch(moe.LayerDims(512, 7168, 2048, 256), 8)  # MFMA path
    with pytest.raises(moe.MoeError):
        moe.layers_one_launch(moe.LayerDims(4, 48, 32, 8), 2)


def test_binding_checks_buffer_sizes(moe):
    """The Python binding compares every tensor's element count with the layer
    sizes (and the quantizer's outputs with its input) before any call, so a
    short buffer never reaches a kernel; these tensors are on the CPU, so the
    check must come before the device check."""
    import torch

    T, d, F, E, k = 4, 64, 64, 8, 2
    x = torch.zeros((T, d), dtype=torch.bfloat16)
    wr = torch.zeros((E, d), dtype=torch.float32)
    p = torch.zeros((E, 3 * d * F // 2), dtype=torch.uint8)
    s = torch.zeros((E, 3 * d * F // 32), dtype=torch.uint8)
    dims = moe.LayerDims(T, d, F, E)
    with pytest.raises(ValueError, match="out has"):
        moe.forward(x, wr, p, s, k, out=torch.zeros((T - 1, d)), dims=dims)
    with pytest.raises(ValueError, match="packed has"):
        moe.forward(x, wr, p[:, :-16].contiguous(), s, k, dims=dims)
    with pytest.raises(ValueError, match="scales has"):
        moe.forward(x, wr, p, s[:-1].contiguous(), k, dims=dims)
    with pytest.raises(ValueError, match="router_w has"):
        moe.forward(x, wr[:-1].contiguous(), p, s, k, dims=dims)
    with pytest.raises(ValueError, match="device tensor"):  # right sizes: only the device is wrong
        moe.forward(x, wr, p, s, k, dims=dims)
    L = 2
    with pytest.raises(ValueError, match="packed has"):
        moe.forward_layers(x, wr.expand(L, E, d).contiguous(), p.expand(L, *p.shape).contiguous()[:, :, :-16]
                           .contiguous(), s.expand(L, *s.shape).contiguous(), k, dims=dims)
    w = torch.zeros((3, 64), dtype=torch.float32)
    with pytest.raises(ValueError, match="packed must be"):
        moe.quantize(w, torch.zeros((3, 31), dtype=torch.uint8), torch.zeros((3, 2), dtype=torch.uint8))
    with pytest.raises(ValueError, match="scales must be"):
        moe.quantize(w, torch.zeros((3, 32), dtype=torch.uint8), torch.zeros((3, 1), dtype=torch.uint8))
    with pytest.raises(ValueError, match="device tensors"):
        moe.quantize(w)
