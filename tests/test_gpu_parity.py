"""GPU parity: the HIP path through the C ABI against the C oracle on the same seeded inputs.

Bars: expert ids, Q8_0 codes and scales, int4 codes and scales, block sums and the
dispatch arrays bit-exact; fp32 outputs within |gpu - oracle| <= max(1e-5 |oracle|, 1e-6).
Tokens the oracle flags as router near-ties (scores within 1e-6 at a selection
boundary) are reported and excluded from id/output equality.
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


def _ws(cfg, T):
    n = moe.moe_workspace_bytes(cfg, T)
    assert n > 0
    return torch.empty(n, dtype=torch.uint8, device=DEV)


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _np(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


# ------------------------------------------------------------------ generator / encoders

def test_synth_gpu_matches_host():
    n = 1 << 20
    t = torch.empty(n, dtype=torch.float32, device=DEV)
    synth.gpu_normal_(t, 7, synth.stream_id(synth.W13, 3, 5), 0.02, start=12345)
    ref = synth.normal(n, 7, synth.stream_id(synth.W13, 3, 5), 0.02, start=12345)
    assert np.array_equal(_np(t).view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("rows,cols", [(64, 32), (128, 256), (192, 96), (4096, 6144)])
def test_quantize_int4_bitexact(rows, cols):
    w = synth.normal(rows * cols, 1, 99, 0.02).reshape(rows, cols)
    w[3] = 0.0
    w[5, 7] = np.float32(0.5)  # a row with one dominant element
    packed = torch.empty(rows * cols // 2, dtype=torch.uint8, device=DEV)
    scales = torch.empty(rows, dtype=torch.float32, device=DEV)
    moe.moe_quantize_int4(_t(w), packed, scales)
    q_gpu = O.unpack_int4_tiled64(_np(packed), rows, cols)
    q_ref, s_ref = O.quant_int4_rows(w)
    assert np.array_equal(_np(scales).view(np.uint32), s_ref.view(np.uint32))
    assert np.array_equal(q_gpu, q_ref)


@pytest.mark.parametrize("n", [32, 32 * 7, 6144 * 3])
def test_quantize_q8_0_bitexact(n):
    x = synth.normal(n, 2, 17, 1.0)
    x[:32] = 0.0
    if n > 64:
        x[32:64] = np.float32(1e-30) * np.arange(32, dtype=np.float32)
        x[64:70] = [127.0, 63.5, -0.5, 1.0, -127.0, 2.5]
    q = torch.empty(n, dtype=torch.int8, device=DEV)
    d = torch.empty(n // 32, dtype=torch.float32, device=DEV)
    moe.moe_quantize_q8_0(_t(x), q, d)
    qr, dr = O.q8_0(x)
    assert np.array_equal(_np(q), qr)
    assert np.array_equal(_np(d).view(np.uint32), dr.view(np.uint32))


# --------------------------------------------------------------------------- router

def _router_case(shape, x, seed=0):
    cfg = config_of(shape)
    T = x.shape[0]
    Wr = synth.router_weights(shape, seed)
    b = synth.router_bias(shape, seed)
    ids = torch.empty((T, shape.top_k), dtype=torch.int32, device=DEV)
    w = torch.empty((T, shape.top_k), dtype=torch.float32, device=DEV)
    fl = torch.empty(T, dtype=torch.uint8, device=DEV)
    moe.moe_router(cfg, _t(x), _t(Wr), _t(b), ids, w, fl, _ws(cfg, T))
    z = O.router_logits(x, Wr)
    rids, rw, rfl = O.route(O.Cfg.of(shape), z, b)
    return _np(ids), _np(w), _np(fl), rids, rw, rfl


@pytest.mark.parametrize("T", [1, 8, 13, 63, 64, 100])
def test_router_tiny(T):
    x = synth.hidden_states(synth.TINY, T, seed=T)
    ids, w, fl, rids, rw, rfl = _router_case(synth.TINY, x)
    clean = (rfl & (O.TIE_EXPERT | O.TIE_GROUP)) == 0
    assert np.array_equal(ids[clean], rids[clean])
    assert within_tol(w[clean], rw[clean])
    assert np.allclose(w.astype(np.float64).sum(1), 2.5, rtol=1e-6)


@pytest.mark.parametrize("T", [1, 32, 192, 256, 300])
def test_router_glm(T):
    """T >= 256 takes the 32-token x 64-expert router tiles; 300 ends in a ragged token block."""
    x = synth.hidden_states(synth.GLM, T, seed=100 + T)
    ids, w, fl, rids, rw, rfl = _router_case(synth.GLM, x)
    clean = (rfl & (O.TIE_EXPERT | O.TIE_GROUP)) == 0
    assert clean.mean() > 0.9
    assert np.array_equal(ids[clean], rids[clean])
    assert within_tol(w[clean], rw[clean])


def test_router_generic_topk_path():
    """E=48 in 4 groups of 12 does not fit the register-resident top-k; the LDS fallback must agree too."""
    sh = synth.Shape(256, 48, 4, 2, 6, 64, 0, 1.5, bias_kind="uniform")
    for T in (5, 70):
        x = synth.hidden_states(sh, T, seed=T)
        ids, w, fl, rids, rw, rfl = _router_case(sh, x)
        clean = (rfl & (O.TIE_EXPERT | O.TIE_GROUP)) == 0
        assert np.array_equal(ids[clean], rids[clean])
        assert within_tol(w[clean], rw[clean])
        assert np.array_equal(fl, rfl)


def test_router_batch_invariance_small_vs_large_kernel():
    """T < 64 and T >= 64 use different kernels; a token's result must not depend on the batch."""
    x = synth.hidden_states(synth.GLM, 80, seed=5)
    ids80, w80, _, _, _, _ = _router_case(synth.GLM, x)
    ids5, w5, _, _, _, _ = _router_case(synth.GLM, x[40:45])
    assert np.array_equal(ids80[40:45], ids5)
    assert np.array_equal(w80[40:45].view(np.uint32), w5.view(np.uint32))


# ------------------------------------------------------------------------- dispatch

# T*K up to 24576 stages the ids in LDS (3072 x 8 is the largest such case), beyond it they are read from
# global memory (3200 x 8); E = 1024 is the largest expert count.
@pytest.mark.parametrize("T,K,E,drop", [(8, 4, 16, 0.0), (1, 8, 256, 0.0), (32, 8, 256, 0.0), (2048, 8, 256, 0.0),
                                        (7, 3, 6, 0.0), (3072, 8, 256, 0.0), (3200, 8, 256, 0.0),
                                        (100, 32, 1024, 0.0), (64, 8, 256, 0.3), (3200, 8, 256, 0.3)])
def test_dispatch_bitexact(T, K, E, drop):
    rng = np.random.default_rng(T + E)
    if E >= 16:
        p = 1.0 / np.arange(1, E + 1) ** 1.1
        ids = np.stack([rng.choice(E, K, replace=False, p=p / p.sum()) for _ in range(T)]).astype(np.int32)
    else:
        ids = rng.integers(0, E, size=(T, K)).astype(np.int32)
    if drop > 0:  # slots dropped by adaptive top-p carry id -1 and belong to no bucket
        ids[rng.random(ids.shape) < drop] = -1
    G = 2 if E % 2 == 0 else 3
    cfg = moe.Config(64, E, G, G, K, 64, 1, 1.0)
    outs = [torch.empty(E, dtype=torch.int32, device=DEV), torch.empty(E + 1, dtype=torch.int32, device=DEV),
            torch.empty(T * K, dtype=torch.int32, device=DEV), torch.empty(T * K, dtype=torch.int32, device=DEV),
            torch.empty(E, dtype=torch.int32, device=DEV), torch.empty(1, dtype=torch.int32, device=DEV)]
    moe.moe_dispatch(cfg, _t(ids), *outs, _ws(cfg, T))
    ref = O.dispatch(ids, E)
    kept = int(ref["offsets"][E])  # sorted_slots past the bucketed slots is unspecified
    for name, t in zip(("counts", "offsets", "sorted_slots", "slot_pos", "unique_ids"), outs[:5]):
        g = _np(t)
        if name == "sorted_slots":
            g, r = g[:kept], ref[name][:kept]
        else:
            r = ref[name]
        assert np.array_equal(g, r), name
    assert int(_np(outs[5])[0]) == ref["n_unique"]


# ------------------------------------------------------------------------ whole layer

@pytest.fixture(scope="module")
def tiny_gpu():
    return GpuLayer(synth.TINY)


@pytest.fixture(scope="module")
def tiny_ref():
    return oracle_layer(synth.TINY)


def _alloc_taps(shape, T, sum_slot=-1):
    H, I, K, E, NS = shape.hidden, shape.inter, shape.top_k, shape.n_experts, shape.n_shared
    R = T * K + NS * T
    b = dict(topk_ids=torch.empty((T, K), dtype=torch.int32, device=DEV),
             topk_w=torch.empty((T, K), dtype=torch.float32, device=DEV),
             near_tie=torch.empty(T, dtype=torch.uint8, device=DEV),
             qx=torch.empty((T, H), dtype=torch.int8, device=DEV),
             dx=torch.empty((T, H // 32), dtype=torch.float32, device=DEV),
             h=torch.empty((R, I), dtype=torch.float32, device=DEV),
             qh=torch.empty((R, I), dtype=torch.int8, device=DEV),
             dh=torch.empty((R, I // 32), dtype=torch.float32, device=DEV),
             e_out=torch.empty((R, H), dtype=torch.float32, device=DEV),
             counts=torch.empty(E, dtype=torch.int32, device=DEV),
             offsets=torch.empty(E + 1, dtype=torch.int32, device=DEV),
             sorted_slots=torch.empty(T * K, dtype=torch.int32, device=DEV),
             slot_pos=torch.empty(T * K, dtype=torch.int32, device=DEV),
             unique_ids=torch.empty(E, dtype=torch.int32, device=DEV),
             n_unique=torch.empty(1, dtype=torch.int32, device=DEV))
    if sum_slot >= 0:
        b["gateup_sums"] = torch.empty((2 * I, H // 32), dtype=torch.int32, device=DEV)
        b["down_sums"] = torch.empty((H, I // 32), dtype=torch.int32, device=DEV)
    return b


def _run_layer(layer, shape, x, gemm_min=0, sum_slot=-1, want_taps=True):
    cfg = config_of(shape, gemm_min)
    T = x.shape[0]
    y = torch.empty((T, shape.hidden), dtype=torch.float32, device=DEV)
    bufs = _alloc_taps(shape, T, sum_slot) if want_taps else {}
    tap = moe.taps(sum_slot, **bufs) if want_taps else None
    moe.moe_layer_forward(cfg, layer.weights(), _t(x), y, _ws(cfg, T), tap)
    torch.cuda.synchronize()
    return _np(y), {k: _np(v) for k, v in bufs.items()}


def _check_all_stages(tiny_gpu, tiny_ref, x, gemm_min, slot):
    sh = synth.TINY
    T, K = x.shape[0], sh.top_k
    y, tp = _run_layer(tiny_gpu, sh, x, gemm_min, sum_slot=slot)
    yr, tr = O.layer_forward(O.Cfg.of(sh), x, tiny_ref)
    assert not (tr["flags"] & (O.TIE_EXPERT | O.TIE_GROUP)).any()
    assert np.array_equal(tp["topk_ids"], tr["ids"])
    assert np.array_equal(tp["topk_w"].view(np.uint32), tr["w"].view(np.uint32))
    assert np.array_equal(tp["near_tie"], tr["flags"])
    assert np.array_equal(tp["qx"], tr["qx"]) and np.array_equal(tp["dx"], tr["dx"])
    assert np.array_equal(tp["h"].view(np.uint32), tr["h"].view(np.uint32))
    assert np.array_equal(tp["qh"], tr["qh"]) and np.array_equal(tp["dh"], tr["dh"])
    assert np.array_equal(tp["e_out"].view(np.uint32), tr["e_out"].view(np.uint32))
    assert within_tol(y, yr)
    assert np.array_equal(y.view(np.uint32), yr.view(np.uint32))
    d = O.dispatch(tr["ids"], sh.n_experts)
    for k in ("counts", "offsets", "sorted_slots", "slot_pos", "unique_ids"):
        assert np.array_equal(tp[k], d[k]), k
    # block sums of one slot (a routed slot, or a shared expert's row): exact int32
    if slot < T * K:
        e = tr["ids"].reshape(-1)[slot]
        q13, q2 = tiny_ref.q13[e], tiny_ref.q2[e]
        t = slot // K
    else:
        s, t = divmod(slot - T * K, T)
        q13, q2 = tiny_ref.sq13[s], tiny_ref.sq2[s]
    S13 = (q13.astype(np.int64) * tr["qx"][t].astype(np.int64)[None]).reshape(2 * sh.inter, -1, 32).sum(2)
    S2 = (q2.astype(np.int64) * tr["qh"][slot].astype(np.int64)[None]).reshape(sh.hidden, -1, 32).sum(2)
    assert np.array_equal(tp["gateup_sums"], S13)
    assert np.array_equal(tp["down_sums"], S2)


@pytest.mark.parametrize("T", [8, 16, 64])
@pytest.mark.parametrize("gemm_min", [1000, 1, 4])
def test_layer_tiny_all_stages(tiny_gpu, tiny_ref, gemm_min, T):
    """Every tap bit-exact against the oracle; the GEMV path (gemm_min=1000, buckets split into chunks of up to 4
    tokens), the MFMA path (gemm_min=1) and a mix give the same bits. The tiny shape has one block per
    accumulation class in gate/up and four empty classes in down; T=8 runs the few-bucket GEMV depth, T=16 the
    many-bucket one. T=64 gives buckets of up to 38 positions: MFMA tiles that are full, part-filled and a
    second tile with a ragged tail."""
    _check_all_stages(tiny_gpu, tiny_ref, synth.hidden_states(synth.TINY, T), gemm_min, 5)


@pytest.mark.parametrize("seed", [0, 3])
@pytest.mark.parametrize("slot", [2, 4])
@pytest.mark.parametrize("gemm_min", [1000, 1, 0])
def test_layer_tiny_one_token(tiny_gpu, tiny_ref, gemm_min, slot, seed):
    """One token: the top-K workgroup writes the dispatch arrays itself (the dispatch launch is skipped), both for
    the GEMV work list (gemm_min 0 or 1000) and for MFMA tiles (gemm_min=1). Every tap bit-exact, block sums of a
    routed slot (2) and of the shared expert (4)."""
    x = synth.hidden_states(synth.TINY, 1, seed=70 + seed)
    _check_all_stages(tiny_gpu, tiny_ref, x, gemm_min, slot)


def test_layer_tiny_batch_invariance(tiny_gpu):
    sh = synth.TINY
    x = synth.hidden_states(sh, 40, seed=9)
    y, _ = _run_layer(tiny_gpu, sh, x, gemm_min=4, want_taps=False)
    for t0, t1 in ((0, 1), (7, 9), (20, 33)):
        ys, _ = _run_layer(tiny_gpu, sh, x[t0:t1], gemm_min=4, want_taps=False)
        assert np.array_equal(ys.view(np.uint32), y[t0:t1].view(np.uint32))
    perm = np.random.default_rng(0).permutation(40)
    yp, _ = _run_layer(tiny_gpu, sh, x[perm], gemm_min=4, want_taps=False)
    assert np.array_equal(yp.view(np.uint32), y[perm].view(np.uint32))


@pytest.mark.parametrize("T", [1, 2, 31, 33, 77])
def test_layer_tiny_ragged_sizes(tiny_gpu, tiny_ref, T):
    sh = synth.TINY
    x = synth.hidden_states(sh, T, seed=50 + T)
    y, tp = _run_layer(tiny_gpu, sh, x, gemm_min=0)
    yr, tr = O.layer_forward(O.Cfg.of(sh), x, tiny_ref)
    clean = (tr["flags"] & (O.TIE_EXPERT | O.TIE_GROUP)) == 0
    assert np.array_equal(tp["topk_ids"][clean], tr["ids"][clean])
    assert within_tol(y[clean], yr[clean])


def test_layer_zero_input(tiny_gpu):
    sh = synth.TINY
    y, tp = _run_layer(tiny_gpu, sh, np.zeros((4, sh.hidden), np.float32))
    assert not y.any()
    assert np.all(tp["topk_w"] == np.float32(sh.rsf / sh.top_k))


def test_layer_rejects_bad_args(tiny_gpu):
    sh = synth.TINY
    cfg = config_of(sh)
    x = torch.zeros((4, sh.hidden), dtype=torch.float32, device=DEV)
    y = torch.empty_like(x)
    ws = _ws(cfg, 4)
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_layer_forward(cfg, tiny_gpu.weights(), x, y, ws[: 1024])
    assert ei.value.rc == moe.MOE_E_WORKSPACE
    bad = config_of(sh)
    bad.hidden = 100
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_layer_forward(bad, tiny_gpu.weights(), x, y, ws)
    assert ei.value.rc == moe.MOE_E_SHAPE
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_layer_forward(cfg, tiny_gpu.weights(), x, y, ws, T=0)
    assert ei.value.rc == moe.MOE_E_SHAPE


SPLIT = synth.Shape(1024, 16, 4, 2, 4, 1024, 1, 2.5, bias_kind="uniform")


@pytest.mark.parametrize("weight_bits", [4, 8])
@pytest.mark.parametrize("slot", [1, 4])
def test_layer_one_token_multi_step(weight_bits, slot):
    """One token at a size whose GEMVs walk several K steps (4 steps of 8 blocks for gate/up and for down, where the
    tiny shape has one): every tap bit-exact against the oracle with int4 and int8 weights, block sums of a routed
    slot (1) and of the shared expert (4) included, so a block lost or reordered between steps fails."""
    sh = SPLIT
    H, I, K, E, NS = sh.hidden, sh.inter, sh.top_k, sh.n_experts, sh.n_shared
    layer = GpuLayer(sh, seed=21, weight_bits=weight_bits)
    ref = oracle_layer(sh, seed=21, weight_bits=weight_bits)
    for seed in (0, 1):
        x = synth.hidden_states(sh, 1, seed=300 + seed)
        cfg = config_of(sh, 0, weight_bits)
        R = K + NS
        bufs = dict(topk_ids=torch.empty((1, K), dtype=torch.int32, device=DEV),
                    topk_w=torch.empty((1, K), dtype=torch.float32, device=DEV),
                    qx=torch.empty((1, H), dtype=torch.int8, device=DEV),
                    h=torch.empty((R, I), dtype=torch.float32, device=DEV),
                    qh=torch.empty((R, I), dtype=torch.int8, device=DEV),
                    e_out=torch.empty((R, H), dtype=torch.float32, device=DEV),
                    gateup_sums=torch.empty((2 * I, H // 32), dtype=torch.int32, device=DEV),
                    down_sums=torch.empty((H, I // 32), dtype=torch.int32, device=DEV))
        y = torch.empty((1, H), dtype=torch.float32, device=DEV)
        moe.moe_layer_forward(cfg, layer.weights(), _t(x), y, _ws(cfg, 1), moe.taps(slot, **bufs))
        g = {k: _np(v) for k, v in bufs.items()}
        yr, tr = O.layer_forward(O.Cfg.of(sh), x, ref)
        assert not (tr["flags"] & (O.TIE_EXPERT | O.TIE_GROUP)).any()
        assert np.array_equal(g["topk_ids"], tr["ids"])
        assert np.array_equal(g["qx"], tr["qx"])
        for k in ("h", "e_out"):
            assert np.array_equal(g[k].view(np.uint32), tr[k].view(np.uint32)), (seed, k)
        assert np.array_equal(g["qh"], tr["qh"])
        assert np.array_equal(_np(y).view(np.uint32), yr.view(np.uint32)), seed
        if slot < K:
            q13, q2 = ref.q13[tr["ids"][0, slot]], ref.q2[tr["ids"][0, slot]]
        else:
            q13, q2 = ref.sq13[slot - K], ref.sq2[slot - K]
        S13 = (q13.astype(np.int64) * tr["qx"][0].astype(np.int64)[None]).reshape(2 * I, -1, 32).sum(2)
        S2 = (q2.astype(np.int64) * tr["qh"][slot].astype(np.int64)[None]).reshape(H, -1, 32).sum(2)
        assert np.array_equal(g["gateup_sums"], S13)
        assert np.array_equal(g["down_sums"], S2)
