"""Per-layer LRU expert cache: routed experts in pinned host memory, an HBM slot pool, copies on a side stream.

Checks, every step: the layer output equals the all-resident layer bit for bit (tier invariance); the hits
and slots equal the oracle's LRU simulator fed the same needed-expert lists; the counters add up."""
import numpy as np
import pytest

from oracle import oracle as O
from synth import synth
from tests.harness import GpuLayer, config_of, host_experts

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import int4_quantized_expert_amd as moe  # noqa: E402

DEV = torch.device("cuda:0")


@pytest.fixture(scope="module")
def tiny():
    layer = GpuLayer(synth.TINY)
    return layer, host_experts(layer)


def _resident_y(layer, cfg, xd, ws):
    y = torch.empty((xd.shape[0], layer.shape.hidden), dtype=torch.float32, device=DEV)
    moe.moe_layer_forward(cfg, layer.weights(), xd, y, ws)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def _run_steps(layer, hx, n_slots, xs, gemm_min=0):
    sh = layer.shape
    cfg = config_of(sh, gemm_min)
    Tmax = max(x.shape[0] for x in xs)
    cache = moe.ExpertCache(cfg, n_slots, Tmax)
    sim = O.LRU(sh.n_experts, n_slots)
    ws = torch.empty(moe.moe_workspace_bytes(cfg, Tmax), dtype=torch.uint8, device=DEV)
    compute, copy = torch.cuda.Stream(), torch.cuda.Stream()
    hits = misses = 0
    for step, x in enumerate(xs):
        xd = torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
        y_ref = _resident_y(layer, cfg, xd, ws)
        y = torch.empty((x.shape[0], sh.hidden), dtype=torch.float32, device=DEV)
        hit, slot = cache.forward(layer.weights(), hx, xd, y, ws, compute, copy, trace=True)
        torch.cuda.synchronize()
        assert np.array_equal(y.cpu().numpy().view(np.uint32), y_ref.view(np.uint32)), step
        needed = np.nonzero(hit >= 0)[0].astype(np.int32)
        r = sim.step(step, needed)
        assert np.array_equal(hit[needed].astype(bool), r["hit"]), step
        assert np.array_equal(slot[needed], r["slot"]), step
        hits += int(r["hit"].sum())
        misses += int((~r["hit"]).sum())
    st = cache.stats()
    assert st["hits"] == hits and st["misses"] == misses and st["steps"] == len(xs)
    assert st["evictions"] == sim.counters()["evictions"]
    per = sh.inter * sh.hidden + 2 * sh.inter * 4 + sh.hidden * sh.inter // 2 + sh.hidden * 4
    assert st["bytes_h2d"] == misses * per
    cache.destroy()
    return st


@pytest.mark.parametrize("n_slots", [4, 1, 16])
def test_cache_tiny_steps(tiny, n_slots):
    layer, (hx, _) = tiny
    xs = [synth.hidden_states(synth.TINY, 8, seed=0, step=s) for s in range(16)]
    st = _run_steps(layer, hx, n_slots, xs)
    if n_slots == 16:
        assert st["evictions"] == 0


def test_cache_tiny_repeat_all_hits(tiny):
    """The same batch twice with room for every expert: the second step is all hits."""
    layer, (hx, _) = tiny
    x = synth.hidden_states(synth.TINY, 8, seed=0, step=3)
    st = _run_steps(layer, hx, 16, [x, x])
    assert st["misses"] > 0 and st["hits"] == st["misses"]


def test_cache_tiny_mfma_and_ragged(tiny):
    """MFMA path (threshold 1) and varying batch sizes through one cache."""
    layer, (hx, _) = tiny
    xs = [synth.hidden_states(synth.TINY, T, seed=1, step=s) for s, T in enumerate([8, 1, 16, 3, 8])]
    _run_steps(layer, hx, 4, xs, gemm_min=1)


def test_cache_rejects_bad_args(tiny):
    layer, (hx, _) = tiny
    cfg = config_of(synth.TINY)
    with pytest.raises(moe.MoeError) as e:
        moe.ExpertCache(cfg, 17, 8)
    assert e.value.rc == moe.MOE_E_ARG
    cache = moe.ExpertCache(cfg, 4, 8)
    ws = torch.empty(moe.moe_workspace_bytes(cfg, 16), dtype=torch.uint8, device=DEV)
    s = torch.cuda.Stream()
    x = torch.zeros((16, 256), dtype=torch.float32, device=DEV)
    y = torch.empty_like(x)
    with pytest.raises(moe.MoeError) as e:
        cache.forward(layer.weights(), hx, x, y, ws, s, torch.cuda.Stream())  # T=16 > max_tokens 8
    assert e.value.rc == moe.MOE_E_SHAPE
    with pytest.raises(moe.MoeError) as e:
        cache.forward(layer.weights(), hx, x[:8], y[:8], ws, s, s)  # one stream for both roles
    assert e.value.rc == moe.MOE_E_ARG
    cache.destroy()


def test_cache_glm_decode32():
    """GLM shape, a 64-slot pool (a quarter of the experts), decode batches of 32."""
    layer = GpuLayer(synth.GLM)
    hx, keep = host_experts(layer)
    xs = [synth.hidden_states(synth.GLM, 32, seed=0, step=s) for s in range(4)]
    st = _run_steps(layer, hx, 64, xs)
    assert st["misses"] > 0
    del keep
