"""Host-side checks of the C ABI (no GPU needed): the library loads, exports every
entry point include/moe.h declares, sizes its workspace, and rejects bad
arguments before touching the device."""
import ctypes
import os
import re

import pytest

import int4_quantized_expert_amd as moe
from int4_quantized_expert_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported():
    names = _declared()
    assert "moe_layer_forward" in names and "moe_router" in names and "moe_dispatch" in names
    lib = ctypes.CDLL(moe.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(moe.EXPORTED)


def test_version_and_errors():
    assert moe.moe_version() >= 10000
    for rc in range(0, -8, -1):
        assert L._lib.moe_strerror(rc)


def _glm(**kw):
    c = moe.Config(6144, 256, 8, 4, 8, 2048, 1, 2.5)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def test_workspace_bytes():
    c = _glm()
    w1, w32, w2048 = (moe.moe_workspace_bytes(c, t) for t in (1, 32, 2048))
    assert 0 < w1 < w32 < w2048
    # dominated by the per-slot fp32 expert outputs: (T*K + T) * H * 4
    assert w2048 >= (2048 * 9) * 6144 * 4
    assert moe.moe_workspace_bytes(c, 0) == 0


@pytest.mark.parametrize("T", [1, 63, 64, 192, 2048])
def test_workspace_covers_every_region(T):
    """Lower bound from what the kernels write per call: router partial sums (T x 16 x E fp64),
    per-slot Q8_0 h codes and scales, per-slot fp32 expert outputs, Q8_0 x, the GEMV work list at its
    worst case (chunks of up to 4 tokens), and the position-blocked x and h operands of the MFMA tiles (whole
    32-position groups) — every batch size, including the large ones."""
    c = _glm()
    E, K, H, I, NS = 256, 8, 6144, 2048, 1
    R = T * K + NS * T
    RP = (R + 31) // 32 * 32
    need = (T * 16 * E * 8 + R * I + R * (I // 32) * 4 + R * H * 4 + T * H + T * (H // 32) * 4
            + ((T * K + NS * T) // 4 + min(E, T * K) + 2 * NS) * 8
            + RP * H + RP * (H // 32) * 4 + RP * I + RP * (I // 32) * 4)
    assert moe.moe_workspace_bytes(c, T) >= need


@pytest.mark.parametrize("bad", [dict(hidden=100), dict(inter=96), dict(n_group=5), dict(topk_group=9),
                                 dict(top_k=40), dict(n_experts=1), dict(n_shared=9), dict(n_group=128, n_experts=128),
                                 dict(routed_scaling_factor=float("nan")), dict(top_k=33)])
def test_invalid_configs_rejected(bad):
    assert moe.moe_workspace_bytes(_glm(**bad), 8) == 0


def test_validation_before_any_device_work():
    c = _glm().c()
    w = L.moe_layer_weights()
    # null weights / inputs are rejected on the host
    rc = L._lib.moe_layer_forward(ctypes.byref(c), ctypes.byref(w), None, 4, None, None, 0, None, None)
    assert rc == L.MOE_E_NULL
    bad = _glm(hidden=100).c()
    rc = L._lib.moe_layer_forward(ctypes.byref(bad), ctypes.byref(w), None, 4, None, None, 0, None, None)
    assert rc == L.MOE_E_SHAPE
    rc = L._lib.moe_quantize_int4(None, 64, 32, None, None, None)
    assert rc == L.MOE_E_NULL
    dummy = ctypes.c_void_p(256)
    rc = L._lib.moe_quantize_int4(dummy, 63, 32, dummy, dummy, None)
    assert rc == L.MOE_E_SHAPE
    rc = L._lib.moe_quantize_q8_0(dummy, 33, dummy, dummy, None)
    assert rc == L.MOE_E_SHAPE
    # workspace too small / misaligned, checked before launch
    x = ctypes.c_void_p(4096)
    wts = L.moe_layer_weights(*([4096] * 10))
    rc = L._lib.moe_layer_forward(ctypes.byref(c), ctypes.byref(wts), x, 4, x, x, 16, None, None)
    assert rc == L.MOE_E_WORKSPACE
    rc = L._lib.moe_layer_forward(ctypes.byref(c), ctypes.byref(wts), x, 4, x, ctypes.c_void_p(4100), 1 << 40,
                                  None, None)
    assert rc == L.MOE_E_WORKSPACE
    rc = L._lib.moe_layer_forward(ctypes.byref(c), ctypes.byref(wts), x, 0, x, x, 1 << 40, None, None)
    assert rc == L.MOE_E_SHAPE


def test_noalloc_validation_before_any_device_work():
    c = _glm().c()
    w = L.moe_layer_weights()
    rc = L._lib.moe_layer_forward_noalloc(ctypes.byref(c), ctypes.byref(w), None, 4, None, None, None)
    assert rc == L.MOE_E_NULL
    bad = _glm(hidden=100).c()
    rc = L._lib.moe_layer_forward_noalloc(ctypes.byref(bad), ctypes.byref(w), None, 4, None, None, None)
    assert rc == L.MOE_E_SHAPE
    x = ctypes.c_void_p(4096)
    wts = L.moe_layer_weights(*([4096] * 10))
    # the GLM shape at 2048 tokens needs more than the fixed array holds
    assert moe.moe_workspace_bytes(_glm(), 2048) > moe.NOALLOC_WORKSPACE_BYTES
    rc = L._lib.moe_layer_forward_noalloc(ctypes.byref(c), ctypes.byref(wts), x, 2048, x, None, None)
    assert rc == L.MOE_E_WORKSPACE
    rc = L._lib.moe_layer_forward_noalloc(ctypes.byref(c), ctypes.byref(wts), x, 0, x, None, None)
    assert rc == L.MOE_E_SHAPE


def test_misaligned_inputs_rejected_before_any_device_work():
    c = _glm().c()
    x = ctypes.c_void_p(4096)
    wts = L.moe_layer_weights(*([4096] * 10))
    rc = L._lib.moe_layer_forward(ctypes.byref(c), ctypes.byref(wts), ctypes.c_void_p(4100), 4, x, x, 1 << 40,
                                  None, None)
    assert rc == L.MOE_E_ARG
    wts2 = L.moe_layer_weights(*([4096, 4096, 4104] + [4096] * 7))
    rc = L._lib.moe_layer_forward(ctypes.byref(c), ctypes.byref(wts2), x, 4, x, x, 1 << 40, None, None)
    assert rc == L.MOE_E_ARG


def test_binding_checks_tensors_before_the_library():
    """The binding hands raw pointers to the library, so it refuses tensors that are not on the GPU, of the
    wrong element type, strided, or smaller than the call touches, and a T above the rows of x."""
    import torch
    c = _glm()
    x = torch.zeros((4, 6144), dtype=torch.float32)
    with pytest.raises(moe.ArgError):
        moe.moe_layer_forward(c, L.moe_layer_weights(), x, x, x)
    with pytest.raises(moe.ArgError):
        moe.moe_quantize_q8_0(x, x, x)
    with pytest.raises(moe.ArgError):
        L._need(x, "x", "f32")  # host tensor
    with pytest.raises(moe.ArgError):
        moe.taps(no_such_tap=x)


def test_tile_converters_validate_before_any_device_work():
    dummy = ctypes.c_void_p(4096)
    for fn in (L._lib.moe_tile_int4, L._lib.moe_tile_int8):
        assert fn(None, 64, 32, dummy, None) == L.MOE_E_NULL
        assert fn(dummy, 64, 32, None, None) == L.MOE_E_NULL
        assert fn(dummy, 63, 32, dummy, None) == L.MOE_E_SHAPE   # rows not whole 64-row tiles
        assert fn(dummy, 64, 48, dummy, None) == L.MOE_E_SHAPE   # cols not whole 32-element blocks
        assert fn(dummy, 0, 32, dummy, None) == L.MOE_E_SHAPE
        assert fn(ctypes.c_void_p(4100), 64, 32, dummy, None) == L.MOE_E_ARG  # 16-byte loads need alignment
        assert fn(dummy, 64, 32, ctypes.c_void_p(4104), None) == L.MOE_E_ARG
    assert L._lib.moe_tile_group_scales(None, 64, 2, dummy, None) == L.MOE_E_NULL
    assert L._lib.moe_tile_group_scales(dummy, 96, 2, dummy, None) == L.MOE_E_SHAPE
    assert L._lib.moe_tile_group_scales(dummy, 64, 0, dummy, None) == L.MOE_E_SHAPE
    import torch
    with pytest.raises(moe.ArgError):
        moe.moe_tile_int4(torch.zeros((64, 16), dtype=torch.uint8), torch.zeros(64 * 16, dtype=torch.uint8))
