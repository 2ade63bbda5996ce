"""Per-layer LRU expert cache: routed experts in pinned host memory, an HBM slot pool, copies on a side stream.

Checks, every step: the layer output equals the all-resident layer bit for bit (tier invariance); the hits
and slots equal the oracle's LRU simulator fed the same needed-expert lists; the counters add up. With the
learning cache: recorded usage equals the simulator's (positions per expert from the oracle's router), and
after a pin call every later step still matches the simulator given the same pins."""
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


def _oracle_counts(sh, x, topp=0.0):
    """Positions routed to each expert, from the oracle's router (the same seeded router weights and bias)."""
    ids, _, _ = O.route(O.Cfg.of(sh, topp=topp), O.router_logits(x, synth.router_weights(sh, 0)),
                        synth.router_bias(sh, 0))
    ids = ids.ravel()
    return np.bincount(ids[ids >= 0], minlength=sh.n_experts)


def _run_steps(layer, hx, n_slots, xs, gemm_min=0, pins=None, usage_check=False, set_usage=None, topp=0.0):
    """pins: {step: n_pin} pin calls made before that step; set_usage: {step: usage} loaded before that step
    into both the cache and the simulator; usage_check: record usage in the simulator from the oracle's
    routing and compare it with the cache's at every pin."""
    sh = layer.shape
    cfg = config_of(sh, gemm_min, layer.weight_bits, layer.group_size, topp)
    Tmax = max(x.shape[0] for x in xs)
    cache = moe.ExpertCache(cfg, n_slots, Tmax)
    sim = O.LRU(sh.n_experts, n_slots)
    ws = torch.empty(moe.moe_workspace_bytes(cfg, Tmax), dtype=torch.uint8, device=DEV)
    compute, copy = torch.cuda.Stream(), torch.cuda.Stream()
    hits = misses = loaded = 0
    for step, x in enumerate(xs):
        if set_usage and step in set_usage:
            cache.set_usage(set_usage[step])
            sim.set_usage(set_usage[step])
        if pins and step in pins:
            if usage_check:
                assert np.array_equal(cache.usage(), sim.usage()), step
            cache.pin_hottest(pins[step], hx, copy)
            loaded += int(sim.pin_hottest(pins[step])["loaded"].sum())
            assert cache.stats()["pinned"] == pins[step]
        xd = torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
        y_ref = _resident_y(layer, cfg, xd, ws)
        y = torch.empty((x.shape[0], sh.hidden), dtype=torch.float32, device=DEV)
        hit, slot = cache.forward(layer.weights(), hx, xd, y, ws, compute, copy, trace=True)
        torch.cuda.synchronize()
        assert np.array_equal(y.cpu().numpy().view(np.uint32), y_ref.view(np.uint32)), step
        needed = np.nonzero(hit >= 0)[0].astype(np.int32)
        r = sim.step(step, needed)
        if usage_check:
            counts = _oracle_counts(sh, x, topp)
            assert np.array_equal(np.nonzero(counts)[0], needed), step
            sim.record_usage(needed, counts[needed])
        assert np.array_equal(hit[needed].astype(bool), r["hit"]), step
        assert np.array_equal(slot[needed], r["slot"]), step
        hits += int(r["hit"].sum())
        misses += int((~r["hit"]).sum())
    st = cache.stats()
    assert st["hits"] == hits and st["misses"] == misses and st["steps"] == len(xs)
    assert st["evictions"] == sim.counters()["evictions"]
    per = sum(t[0].numel() * t.element_size() for t in (layer.w13, layer.s13, layer.w2, layer.s2))
    wb, G = layer.weight_bits, layer.group_size
    nsc = (2 * sh.inter * sh.hidden // G + sh.hidden * sh.inter // G) if G else 2 * sh.inter + sh.hidden
    assert per == sh.inter * sh.hidden * wb // 4 + sh.hidden * sh.inter * wb // 8 + 4 * nsc
    assert st["bytes_h2d"] == (misses + loaded) * per
    if usage_check:
        assert np.array_equal(cache.usage(), sim.usage())
    cache.destroy()
    return st


@pytest.fixture(scope="module")
def tiny8():
    layer = GpuLayer(synth.TINY, weight_bits=8)
    return layer, host_experts(layer)


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


def test_cache_tiny_parts_not_in_slot_order(tiny):
    """Host parts in another order (w2, s2, w13, s13): misses move in four transfers; results and counts as
    with one transfer."""
    layer, _ = tiny
    hx, _keep = host_experts(layer, order=(2, 3, 0, 1))
    xs = [synth.hidden_states(synth.TINY, T, seed=8, step=s) for s, T in enumerate([8, 16, 3, 8])]
    _run_steps(layer, hx, 4, xs, gemm_min=0)
    _run_steps(layer, hx, 4, xs, gemm_min=1, pins={2: 2}, usage_check=True)


@pytest.mark.parametrize("gemm_min", [0, 1])
def test_cache_tiny_topp(tiny, gemm_min):
    """Adaptive top-p through the cache: only kept slots' experts are needed, usage counts kept positions."""
    layer, (hx, _) = tiny
    xs = [synth.hidden_states(synth.TINY, T, seed=7, step=s) for s, T in enumerate([8, 16, 3, 8, 1, 8])]
    _run_steps(layer, hx, 4, xs, gemm_min=gemm_min, pins={3: 2}, usage_check=True, topp=0.6)


@pytest.mark.parametrize("gemm_min", [0, 1])
def test_cache_tiny_grouped_scales(gemm_min):
    """int4 experts with group scales through the cache: the slots carry the larger scale arrays."""
    layer = GpuLayer(synth.TINY, group_size=32)
    hx, _keep = host_experts(layer)
    xs = [synth.hidden_states(synth.TINY, T, seed=6, step=s) for s, T in enumerate([8, 16, 3, 8, 1])]
    _run_steps(layer, hx, 4, xs, gemm_min=gemm_min, pins={3: 1}, usage_check=True)


@pytest.mark.parametrize("gemm_min", [0, 1])
def test_cache_tiny_int8_weights(tiny8, gemm_min):
    """int8 experts through the cache: slots sized for int8, copies of the int8 bytes, output equal to the
    all-resident int8 layer; with pins."""
    layer, (hx, _) = tiny8
    xs = [synth.hidden_states(synth.TINY, T, seed=4, step=s) for s, T in enumerate([8, 1, 16, 3, 8, 8, 5])]
    _run_steps(layer, hx, 4, xs, gemm_min=gemm_min, pins={4: 2}, usage_check=True)


@pytest.mark.parametrize("n_slots,pins", [(6, {8: 3}), (4, {5: 2, 10: 0, 12: 3}), (1, {6: 0})])
def test_cache_tiny_learning_pins(tiny, n_slots, pins):
    """Usage recorded over steps equals the simulator's; pinning the most used experts (and releasing pins)
    leaves every later step equal to the simulator with the same pins, and the output bit-exact."""
    layer, (hx, _) = tiny
    xs = [synth.hidden_states(synth.TINY, 8, seed=2, step=s) for s in range(16)]
    st = _run_steps(layer, hx, n_slots, xs, pins=pins, usage_check=True)
    assert st["pinned"] == pins[max(pins)]


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
    with pytest.raises(moe.MoeError) as e:
        cache.pin_hottest(4, hx, s)  # at least one slot must stay unpinned
    assert e.value.rc == moe.MOE_E_ARG
    with pytest.raises(moe.MoeError) as e:
        cache.set_usage(np.full(16, -1, np.int64))
    assert e.value.rc == moe.MOE_E_ARG
    cache.destroy()


def test_cache_glm_decode32():
    """GLM shape, a 64-slot pool (a quarter of the experts), decode batches of 32."""
    layer = GpuLayer(synth.GLM)
    hx, keep = host_experts(layer)
    xs = [synth.hidden_states(synth.GLM, 32, seed=0, step=s) for s in range(4)]
    st = _run_steps(layer, hx, 64, xs)
    assert st["misses"] > 0
    # learning cache at the GLM shape: 48 of the 64 slots pinned from a seeded usage profile
    usage = np.random.default_rng(5).zipf(1.2, size=256).astype(np.int64)
    st = _run_steps(layer, hx, 64, xs + xs[:2], set_usage={2: usage}, pins={2: 48})
    assert st["pinned"] == 48
    del keep
