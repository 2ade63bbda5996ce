"""moe_layer_forward_noalloc against moe_layer_forward, through the C ABI.

The entry point for callers that cannot allocate runs the same kernels in the
library's fixed device array; its outputs must equal moe_layer_forward's bit for
bit. Each case makes two calls in a row on that array, the second with fewer
tokens, so that the second call runs over what the first one left behind.
"""
import ctypes

import numpy as np
import pytest

from synth import synth
from tests.harness import GpuLayer, config_of

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import int4_quantized_expert_amd as moe  # noqa: E402

DEV = torch.device("cuda:0")


def _pair(cfg, layer, x):
    """(y of moe_layer_forward, y and routing ids of moe_layer_forward_noalloc) for the tokens x."""
    T = x.shape[0]
    H = cfg.hidden
    ws = torch.empty(moe.moe_workspace_bytes(cfg, T), dtype=torch.uint8, device=DEV)
    y_ref = torch.empty((T, H), dtype=torch.float32, device=DEV)
    ids_ref = torch.empty((T, cfg.top_k), dtype=torch.int32, device=DEV)
    moe.moe_layer_forward(cfg, layer.weights(), x, y_ref, ws, moe.taps(topk_ids=ids_ref))
    y = torch.full((T, H), float("nan"), dtype=torch.float32, device=DEV)
    ids = torch.full((T, cfg.top_k), -7, dtype=torch.int32, device=DEV)
    moe.moe_layer_forward_noalloc(cfg, layer.weights(), x, y, moe.taps(topk_ids=ids))
    torch.cuda.synchronize()
    return y_ref.cpu().numpy(), ids_ref.cpu().numpy(), y.cpu().numpy(), ids.cpu().numpy()


def _x(shape, T, step):
    return torch.from_numpy(synth.hidden_states(shape, T, seed=0, step=step)).to(DEV)


@pytest.mark.parametrize("shape_name,sizes", [("TINY", (64, 5)), ("GLM", (192, 32)), ("GLM", (32, 1))])
def test_noalloc_equals_layer_forward_twice(shape_name, sizes):
    shape = getattr(synth, shape_name)
    cfg = config_of(shape)
    layer = _layer(shape_name)
    for i, T in enumerate(sizes):
        assert moe.moe_workspace_bytes(cfg, T) <= moe.NOALLOC_WORKSPACE_BYTES
        print(f"noalloc case {shape_name} T={T} call {i}", flush=True)
        y_ref, ids_ref, y, ids = _pair(cfg, layer, _x(shape, T, 100 + i))
        assert np.array_equal(ids, ids_ref)
        assert np.array_equal(y.view(np.uint32), y_ref.view(np.uint32)), (shape_name, T)


def test_noalloc_rejects_what_does_not_fit_before_any_work():
    cfg = config_of(synth.GLM)
    T = 2048
    assert moe.moe_workspace_bytes(cfg, T) > moe.NOALLOC_WORKSPACE_BYTES
    layer = _layer("GLM")
    x = _x(synth.GLM, 8, 0)
    y = torch.zeros((8, synth.GLM.hidden), dtype=torch.float32, device=DEV)
    c = cfg.c()
    w = layer.weights()
    # straight through the C ABI: the binding itself refuses T above the rows of x
    rc = moe._lib._lib.moe_layer_forward_noalloc(ctypes.byref(c), ctypes.byref(w), moe._lib._ptr(x), T,
                                                 moe._lib._ptr(y), None, moe._lib._stream(None))
    assert rc == moe.MOE_E_WORKSPACE
    with pytest.raises(moe.ArgError):
        moe.moe_layer_forward_noalloc(cfg, w, x, y, T=T)
    torch.cuda.synchronize()
    assert not bool(y.any())  # nothing was enqueued


_LAYERS = {}


def _layer(name):
    if name not in _LAYERS:
        _LAYERS.clear()
        _LAYERS[name] = GpuLayer(getattr(synth, name))
    return _LAYERS[name]
