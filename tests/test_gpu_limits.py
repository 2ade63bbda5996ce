"""GPU parity at the largest sizes the library accepts: hidden 16384 with four
shared experts, inter 16384, and 1024 experts in 64 groups with top-32. Every
tap is bit-exact against the oracle on the GEMV path, the MFMA path and the
default split, for a batch with MFMA-sized buckets (T = 40) and a small one
(T = 7). The inputs have no router near-ties.
"""
import numpy as np
import pytest

from oracle import oracle as O
from synth import synth
from tests.harness import GpuLayer, config_of, oracle_layer

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import int4_quantized_expert_amd as moe  # noqa: E402

DEV = torch.device("cuda:0")

SHAPES = {
    "max_hidden": synth.Shape(16384, 16, 4, 2, 4, 128, 4, 2.5, bias_kind="uniform"),
    "max_inter": synth.Shape(128, 16, 4, 2, 4, 16384, 1, 2.5, bias_kind="uniform"),
    "max_experts": synth.Shape(256, 1024, 64, 8, 32, 64, 1, 2.5, bias_kind="uniform"),
}
_LAYERS = {}


def _layer(name):
    if name not in _LAYERS:
        sh = SHAPES[name]
        _LAYERS.clear()  # one shape's device layer and oracle copy at a time
        _LAYERS[name] = (GpuLayer(sh), oracle_layer(sh))
    return _LAYERS[name]


def _run(layer, x, gemm_min):
    sh = layer.shape
    H, I, K, NS = sh.hidden, sh.inter, sh.top_k, layer.NS
    cfg = config_of(sh, gemm_min)
    T = x.shape[0]
    R = T * K + NS * T
    y = torch.empty((T, H), dtype=torch.float32, device=DEV)
    bufs = dict(topk_ids=torch.empty((T, K), dtype=torch.int32, device=DEV),
                topk_w=torch.empty((T, K), dtype=torch.float32, device=DEV),
                qx=torch.empty((T, H), dtype=torch.int8, device=DEV),
                dx=torch.empty((T, H // 32), dtype=torch.float32, device=DEV),
                h=torch.empty((R, I), dtype=torch.float32, device=DEV),
                qh=torch.empty((R, I), dtype=torch.int8, device=DEV),
                dh=torch.empty((R, I // 32), dtype=torch.float32, device=DEV),
                e_out=torch.empty((R, H), dtype=torch.float32, device=DEV))
    ws = torch.empty(moe.moe_workspace_bytes(cfg, T), dtype=torch.uint8, device=DEV)
    moe.moe_layer_forward(cfg, layer.weights(), torch.from_numpy(np.ascontiguousarray(x)).to(DEV), y, ws,
                          moe.taps(-1, **bufs))
    torch.cuda.synchronize()
    return y.cpu().numpy(), {k: v.cpu().numpy() for k, v in bufs.items()}


@pytest.mark.parametrize("name", list(SHAPES))
@pytest.mark.parametrize("T,seed", [(40, 3), (7, 4)])
@pytest.mark.parametrize("gemm_min", [0, 1000, 1])
def test_limits_all_taps_bitexact(name, T, seed, gemm_min):
    layer, ref = _layer(name)
    sh = SHAPES[name]
    x = synth.hidden_states(sh, T, seed=seed)
    y, tp = _run(layer, x, gemm_min)
    yr, tr = O.layer_forward(O.Cfg.of(sh), x, ref)
    assert not (tr["flags"] & (O.TIE_EXPERT | O.TIE_GROUP)).any()
    assert np.array_equal(tp["topk_ids"], tr["ids"])
    assert np.array_equal(tp["topk_w"].view(np.uint32), tr["w"].view(np.uint32))
    assert np.array_equal(tp["qx"], tr["qx"]) and np.array_equal(tp["dx"].view(np.uint32), tr["dx"].view(np.uint32))
    assert np.array_equal(tp["h"].view(np.uint32), tr["h"].view(np.uint32))
    assert np.array_equal(tp["qh"], tr["qh"]) and np.array_equal(tp["dh"].view(np.uint32), tr["dh"].view(np.uint32))
    assert np.array_equal(tp["e_out"].view(np.uint32), tr["e_out"].view(np.uint32))
    assert np.array_equal(y.view(np.uint32), yr.view(np.uint32))


def test_limits_rejects_past_the_maximum():
    big_h = synth.Shape(16384 + 64, 16, 4, 2, 4, 128, 1, 2.5)
    big_e = synth.Shape(256, 1088, 64, 8, 32, 64, 1, 2.5)
    big_k = synth.Shape(256, 1024, 64, 8, 33, 64, 1, 2.5)
    big_ns = synth.Shape(256, 16, 4, 2, 4, 128, 5, 2.5)
    for sh in (big_h, big_e, big_k, big_ns):
        assert moe.moe_workspace_bytes(config_of(sh), 8) == 0, sh
