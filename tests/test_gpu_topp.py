"""GPU parity for adaptive expert top-p (moe_config.topp in (0, 1); "Show HN: 느린
컴퓨터에서 GLM 5.2 실행하기", useful options: --topp 0.7). A token keeps only the
slots, by normalised weight descending, while the fp64 sum of the kept weights is
below topp; the kept weights are renormalised; dropped slots have id -1, weight 0,
no bucket and no share in the combine.

Router ids (with -1) and weights, the dispatch arrays and every tap of the kept
slots are bit-exact against the oracle on the tiny layer (GEMV, MFMA and mixed
paths); at the GLM-5.2 shape sampled tokens are checked one at a time and the
paths agree; the expert cache stays bit-exact against the resident layer.
"""
import numpy as np
import pytest

from oracle import oracle as O
from synth import synth
from tests.harness import GpuLayer, config_of, oracle_layer, oracle_tokens, within_tol

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import int4_quantized_expert_amd as moe  # noqa: E402

DEV = torch.device("cuda:0")


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _np(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


# (shape, T, topp, whether the oracle drops any slot); TINY T = 7 at 0.8 keeps every slot
@pytest.mark.parametrize("shape_name,T,topp,drops", [("TINY", 40, 0.5, True), ("TINY", 7, 0.8, False),
                                                     ("TINY", 7, 0.6, True), ("GLM", 32, 0.7, True),
                                                     ("GLM", 300, 0.7, True), ("GLM", 5, 0.3, True)])
def test_router_topp_bitexact(shape_name, T, topp, drops):
    sh = getattr(synth, shape_name)
    cfg = config_of(sh, 0, 4, 0, topp)
    x = synth.hidden_states(sh, T, seed=60 + T)
    Wr, bias = synth.router_weights(sh), synth.router_bias(sh)
    ids = torch.empty((T, sh.top_k), dtype=torch.int32, device=DEV)
    w = torch.empty((T, sh.top_k), dtype=torch.float32, device=DEV)
    fl = torch.empty(T, dtype=torch.uint8, device=DEV)
    ws = torch.empty(moe.moe_workspace_bytes(cfg, T), dtype=torch.uint8, device=DEV)
    moe.moe_router(cfg, _t(x), _t(Wr), _t(bias), ids, w, fl, ws)
    ir, wr, fr = O.route(O.Cfg.of(sh, topp=topp), O.router_logits(x, Wr), bias)
    clean = (fr & (O.TIE_EXPERT | O.TIE_GROUP)) == 0
    assert np.array_equal(_np(fl), fr)
    assert np.array_equal(_np(ids)[clean], ir[clean])
    assert np.array_equal(_np(w)[clean].view(np.uint32), wr[clean].view(np.uint32))
    assert (ir < 0).any() == drops and (ir >= 0).any(1).all()


def test_dispatch_with_dropped_slots_bitexact():
    sh = synth.GLM
    T, K, E = 64, sh.top_k, sh.n_experts
    rng = np.random.default_rng(3)
    ids = rng.integers(0, E, (T, K)).astype(np.int32)
    ids[rng.random((T, K)) < 0.4] = -1
    cfg = config_of(sh)
    d = O.dispatch(ids, E)
    out = dict(counts=torch.empty(E, dtype=torch.int32, device=DEV),
               offsets=torch.empty(E + 1, dtype=torch.int32, device=DEV),
               sorted_slots=torch.full((T * K,), -1, dtype=torch.int32, device=DEV),
               slot_pos=torch.empty(T * K, dtype=torch.int32, device=DEV),
               unique_ids=torch.empty(E, dtype=torch.int32, device=DEV),
               n_unique=torch.empty(1, dtype=torch.int32, device=DEV))
    ws = torch.empty(moe.moe_workspace_bytes(cfg, T), dtype=torch.uint8, device=DEV)
    moe.moe_dispatch(cfg, _t(ids), out["counts"], out["offsets"], out["sorted_slots"], out["slot_pos"],
                     out["unique_ids"], out["n_unique"], ws)
    g = {k: _np(v) for k, v in out.items()}
    n = int(d["offsets"][E])
    for k in ("counts", "offsets", "slot_pos", "unique_ids"):
        assert np.array_equal(g[k], d[k]), k
    assert np.array_equal(g["sorted_slots"][:n], d["sorted_slots"][:n])
    assert int(g["n_unique"][0]) == d["n_unique"]


# ------------------------------------------------------------------ tiny layer

@pytest.fixture(scope="module")
def tiny():
    return GpuLayer(synth.TINY), oracle_layer(synth.TINY)


def _run(layer, x, topp, gemm_min=0):
    sh = layer.shape
    H, I, K, NS = sh.hidden, sh.inter, sh.top_k, layer.NS
    cfg = config_of(sh, gemm_min, 4, 0, topp)
    T = x.shape[0]
    R = T * K + NS * T
    y = torch.empty((T, H), dtype=torch.float32, device=DEV)
    bufs = dict(topk_ids=torch.empty((T, K), dtype=torch.int32, device=DEV),
                topk_w=torch.empty((T, K), dtype=torch.float32, device=DEV),
                h=torch.zeros((R, I), dtype=torch.float32, device=DEV),
                qh=torch.zeros((R, I), dtype=torch.int8, device=DEV),
                e_out=torch.zeros((R, H), dtype=torch.float32, device=DEV),
                counts=torch.empty(sh.n_experts, dtype=torch.int32, device=DEV),
                n_unique=torch.empty(1, dtype=torch.int32, device=DEV))
    ws = torch.empty(moe.moe_workspace_bytes(cfg, T), dtype=torch.uint8, device=DEV)
    moe.moe_layer_forward(cfg, layer.weights(), _t(x), y, ws, moe.taps(-1, **bufs))
    torch.cuda.synchronize()
    return _np(y), {k: _np(v) for k, v in bufs.items()}


@pytest.mark.parametrize("gemm_min", [1000, 1, 4])
@pytest.mark.parametrize("topp", [0.5, 0.75])
def test_topp_layer_tiny_all_stages(tiny, gemm_min, topp):
    layer, ref = tiny
    sh = synth.TINY
    x = synth.hidden_states(sh, 24, seed=70)
    y, tp = _run(layer, x, topp, gemm_min)
    yr, tr = O.layer_forward(O.Cfg.of(sh, topp=topp), x, ref)
    assert not (tr["flags"] & (O.TIE_EXPERT | O.TIE_GROUP)).any()
    assert np.array_equal(tp["topk_ids"], tr["ids"])
    assert np.array_equal(tp["topk_w"].view(np.uint32), tr["w"].view(np.uint32))
    kept = np.concatenate([tr["ids"].ravel() >= 0, np.ones(24 * layer.NS, bool)])
    assert (~kept).any()
    for k in ("h", "e_out"):
        assert np.array_equal(tp[k][kept].view(np.uint32), tr[k][kept].view(np.uint32)), k
    assert np.array_equal(tp["qh"][kept], tr["qh"][kept])
    assert np.array_equal(y.view(np.uint32), yr.view(np.uint32))
    assert np.array_equal(tp["counts"], np.bincount(tr["ids"][tr["ids"] >= 0], minlength=sh.n_experts))


@pytest.mark.parametrize("gemm_min", [1000, 1])
def test_topp_layer_tiny_one_token(tiny, gemm_min):
    """One token at a time with adaptive top-p: the top-K workgroup dispatches only the kept slots (dropped slots
    have no position and no share in the combine)."""
    layer, ref = tiny
    sh = synth.TINY
    dropped = 0
    for seed in range(8):
        x = synth.hidden_states(sh, 1, seed=200 + seed)
        y, tp = _run(layer, x, 0.5, gemm_min)
        yr, tr = O.layer_forward(O.Cfg.of(sh, topp=0.5), x, ref)
        if tr["flags"][0] & (O.TIE_EXPERT | O.TIE_GROUP):
            continue
        assert np.array_equal(tp["topk_ids"], tr["ids"])
        assert np.array_equal(tp["topk_w"].view(np.uint32), tr["w"].view(np.uint32))
        kept = np.concatenate([tr["ids"].ravel() >= 0, np.ones(layer.NS, bool)])
        dropped += int((~kept).sum())
        for k in ("h", "e_out"):
            assert np.array_equal(tp[k][kept].view(np.uint32), tr[k][kept].view(np.uint32)), (seed, k)
        assert np.array_equal(y.view(np.uint32), yr.view(np.uint32)), seed
        assert np.array_equal(tp["counts"], np.bincount(tr["ids"][tr["ids"] >= 0], minlength=sh.n_experts))
        assert tp["n_unique"][0] == (tr["ids"] >= 0).sum()
    assert dropped > 0


def test_topp_off_values_equal_no_topp(tiny):
    layer, _ = tiny
    x = synth.hidden_states(synth.TINY, 16, seed=71)
    y0, _ = _run(layer, x, 0.0)
    for off in (1.0, -0.5, 2.0):
        y1, _ = _run(layer, x, off)
        assert np.array_equal(y0.view(np.uint32), y1.view(np.uint32))


def test_topp_rejects_nan(tiny):
    layer, _ = tiny
    sh = synth.TINY
    cfg = config_of(sh, 0, 4, 0, float("nan"))
    assert moe.moe_workspace_bytes(cfg, 4) == 0


# ------------------------------------------------------------------ GLM-5.2 layer shape

SH = synth.GLM


@pytest.fixture(scope="module")
def glm():
    return GpuLayer(SH)


def _forward(layer, x, topp, gemm_min=0):
    cfg = config_of(SH, gemm_min, 4, 0, topp)
    T = x.shape[0]
    ws = torch.empty(moe.moe_workspace_bytes(cfg, T), dtype=torch.uint8, device=DEV)
    y = torch.empty((T, SH.hidden), dtype=torch.float32, device=DEV)
    nu = torch.empty(1, dtype=torch.int32, device=DEV)
    moe.moe_layer_forward(cfg, layer.weights(), _t(x), y, ws, moe.taps(-1, n_unique=nu))
    return _np(y), int(_np(nu)[0])


@pytest.mark.parametrize("T,tokens", [(32, [0, 17, 31]), (192, [0, 100, 191])])
def test_topp_glm_sampled(glm, T, tokens):
    x = synth.hidden_states(SH, T, seed=0, step=7)
    y, nu = _forward(glm, x, 0.7)
    _, nu_all = _forward(glm, x, 0.0)
    assert nu <= nu_all
    ref = oracle_tokens(SH, x, tokens, topp=0.7)
    ties = []
    for t in tokens:
        r = ref[t]
        if r["flags"] & (O.TIE_EXPERT | O.TIE_GROUP):
            ties.append(t)
            continue
        assert within_tol(y[t], r["y"]), (t, float(np.max(np.abs(y[t] - r["y"]))))
    assert len(ties) < len(tokens)


def test_topp_glm_paths_agree(glm):
    x = synth.hidden_states(SH, 64, seed=0, step=8)
    y0, _ = _forward(glm, x, 0.7)
    assert np.array_equal(y0.view(np.uint32), _forward(glm, x, 0.7, gemm_min=1000)[0].view(np.uint32))
    assert np.array_equal(y0.view(np.uint32), _forward(glm, x, 0.7, gemm_min=1)[0].view(np.uint32))
