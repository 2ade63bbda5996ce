"""GPU parity for grouped int4 weight scales (group_size G > 0): one fp32 scale per
G elements along each row, the quality fix the colibrì pages point to ("Colibri:
25GB RAM을 탑재한 노트북에서 744B AI 모델 실행하기", section on the quality cost of
int4). The dot scales each block's exact sum by fp32(d_b * s_group(b)) in one
ascending running sum, with no row scale.

The encoder (codes and tiled scales) is bit-exact against the oracle's; every tap
of the tiny layer is bit-exact on the GEMV, MFMA and mixed paths for G = 32, 64
and 128; at the GLM-5.2 layer shape sampled tokens are checked one at a time
(outputs within |gpu - oracle| <= max(1e-5 |oracle|, 1e-6)) and the three paths
give the same bits.
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


@pytest.mark.parametrize("rows,cols,group", [(64, 32, 32), (128, 256, 64), (192, 384, 128), (4096, 6144, 32),
                                             (2048, 6144, 256)])
def test_quantize_int4_grouped_bitexact(rows, cols, group):
    w = synth.normal(rows * cols, 3, 97, 0.02).reshape(rows, cols)
    w[3] = 0.0
    w[5, 7] = np.float32(0.5)
    w[6, :4] = [7.0, -3.5, 0.5, -0.5]
    packed = torch.empty(rows * cols // 2, dtype=torch.uint8, device=DEV)
    scales = torch.empty(rows * cols // group, dtype=torch.float32, device=DEV)
    moe.moe_quantize_int4_grouped(_t(w), group, packed, scales)
    q_gpu = O.unpack_int4_tiled64(_np(packed), rows, cols)
    s_gpu = O.unpack_scales_tiled64(_np(scales), rows, cols // group)
    q_ref, s_ref = O.quant_int4_grouped(w, group)
    assert np.array_equal(s_gpu.view(np.uint32), s_ref.view(np.uint32))
    assert np.array_equal(q_gpu, q_ref)


def test_quantize_int4_grouped_rejects_bad_args():
    w = torch.zeros((64, 96), dtype=torch.float32, device=DEV)
    packed = torch.empty(64 * 48, dtype=torch.uint8, device=DEV)
    scales = torch.empty(64 * 3, dtype=torch.float32, device=DEV)
    for g, rc in ((48, moe.MOE_E_ARG), (96, moe.MOE_E_ARG), (0, moe.MOE_E_ARG), (64, moe.MOE_E_SHAPE)):
        with pytest.raises(moe.MoeError) as ei:
            moe.moe_quantize_int4_grouped(w, g, packed, scales)
        assert ei.value.rc == rc, g


# ------------------------------------------------------------------ tiny layer

_TINY = {}


def _tiny(G):
    if G not in _TINY:
        _TINY[G] = (GpuLayer(synth.TINY, group_size=G), oracle_layer(synth.TINY, group_size=G))
    return _TINY[G]


def _run(layer, x, gemm_min=0, sum_slot=-1, want_taps=True):
    sh = layer.shape
    H, I, K, NS = sh.hidden, sh.inter, sh.top_k, layer.NS
    cfg = config_of(sh, gemm_min, 4, layer.group_size)
    T = x.shape[0]
    R = T * K + NS * T
    y = torch.empty((T, H), dtype=torch.float32, device=DEV)
    bufs = {}
    if want_taps:
        bufs = dict(topk_ids=torch.empty((T, K), dtype=torch.int32, device=DEV),
                    qx=torch.empty((T, H), dtype=torch.int8, device=DEV),
                    dx=torch.empty((T, H // 32), dtype=torch.float32, device=DEV),
                    h=torch.empty((R, I), dtype=torch.float32, device=DEV),
                    qh=torch.empty((R, I), dtype=torch.int8, device=DEV),
                    dh=torch.empty((R, I // 32), dtype=torch.float32, device=DEV),
                    e_out=torch.empty((R, H), dtype=torch.float32, device=DEV))
        if sum_slot >= 0:
            bufs["gateup_sums"] = torch.empty((2 * I, H // 32), dtype=torch.int32, device=DEV)
            bufs["down_sums"] = torch.empty((H, I // 32), dtype=torch.int32, device=DEV)
    tap = moe.taps(sum_slot, **bufs) if want_taps else None
    ws = torch.empty(moe.moe_workspace_bytes(cfg, T), dtype=torch.uint8, device=DEV)
    moe.moe_layer_forward(cfg, layer.weights(), _t(x), y, ws, tap)
    torch.cuda.synchronize()
    return _np(y), {k: _np(v) for k, v in bufs.items()}


@pytest.mark.parametrize("T", [1, 16, 64])
@pytest.mark.parametrize("G", [32, 64, 128])
@pytest.mark.parametrize("gemm_min", [1000, 1, 4])
def test_grouped_layer_tiny_all_stages(G, gemm_min, T):
    """Every tap bit-exact against the oracle with group scales, on the GEMV path, the MFMA path (T = 64: buckets
    past one 32-position tile) and a mix; T = 1 takes the one-token dispatch."""
    layer, ref = _tiny(G)
    sh = synth.TINY
    K = sh.top_k
    x = synth.hidden_states(sh, T, seed=31)
    slot = 6 if T > 1 else 2
    y, tp = _run(layer, x, gemm_min, sum_slot=slot)
    yr, tr = O.layer_forward(O.Cfg.of(sh, group=G), x, ref)
    assert not (tr["flags"] & (O.TIE_EXPERT | O.TIE_GROUP)).any()
    assert np.array_equal(tp["topk_ids"], tr["ids"])
    assert np.array_equal(tp["qx"], tr["qx"]) and np.array_equal(tp["dx"], tr["dx"])
    assert np.array_equal(tp["h"].view(np.uint32), tr["h"].view(np.uint32))
    assert np.array_equal(tp["qh"], tr["qh"]) and np.array_equal(tp["dh"], tr["dh"])
    assert np.array_equal(tp["e_out"].view(np.uint32), tr["e_out"].view(np.uint32))
    assert np.array_equal(y.view(np.uint32), yr.view(np.uint32))
    e = tr["ids"].reshape(-1)[slot]
    S13 = (ref.q13[e].astype(np.int64) * tr["qx"][slot // K].astype(np.int64)[None]).reshape(2 * sh.inter, -1,
                                                                                              32).sum(2)
    S2 = (ref.q2[e].astype(np.int64) * tr["qh"][slot].astype(np.int64)[None]).reshape(sh.hidden, -1, 32).sum(2)
    assert np.array_equal(tp["gateup_sums"], S13)
    assert np.array_equal(tp["down_sums"], S2)


@pytest.mark.parametrize("T", [1, 33, 77])
def test_grouped_layer_tiny_ragged(T):
    layer, ref = _tiny(32)
    sh = synth.TINY
    x = synth.hidden_states(sh, T, seed=90 + T)
    y, tp = _run(layer, x, gemm_min=0)
    yr, tr = O.layer_forward(O.Cfg.of(sh, group=32), x, ref)
    clean = (tr["flags"] & (O.TIE_EXPERT | O.TIE_GROUP)) == 0
    assert np.array_equal(tp["topk_ids"][clean], tr["ids"][clean])
    assert within_tol(y[clean], yr[clean])


def test_grouped_config_rejected():
    layer, _ = _tiny(32)
    sh = synth.TINY
    x = torch.zeros((4, sh.hidden), dtype=torch.float32, device=DEV)
    y = torch.empty_like(x)
    ws = torch.empty(1 << 22, dtype=torch.uint8, device=DEV)
    for wb, G, rc in ((8, 32, moe.MOE_E_ARG), (4, 48, moe.MOE_E_ARG), (4, 96, moe.MOE_E_ARG),
                      (4, 256, moe.MOE_E_SHAPE)):
        cfg = config_of(sh, 0, wb, G)
        assert moe.moe_workspace_bytes(cfg, 4) == 0
        with pytest.raises(moe.MoeError) as ei:
            moe.moe_layer_forward(cfg, layer.weights(), x, y, ws)
        assert ei.value.rc == rc, (wb, G)


# ------------------------------------------------------------------ GLM-5.2 layer shape

SH = synth.GLM


@pytest.fixture(scope="module")
def glm_g32():
    return GpuLayer(SH, group_size=32)


def _forward(layer, x, gemm_min=0):
    cfg = config_of(SH, gemm_min, 4, layer.group_size)
    T = x.shape[0]
    ws = torch.empty(moe.moe_workspace_bytes(cfg, T), dtype=torch.uint8, device=DEV)
    y = torch.empty((T, SH.hidden), dtype=torch.float32, device=DEV)
    moe.moe_layer_forward(cfg, layer.weights(), _t(x), y, ws)
    return _np(y)


def _check(layer, x, tokens):
    y = _forward(layer, x)
    ref = oracle_tokens(SH, x, tokens, group_size=layer.group_size)
    ties = []
    for t in tokens:
        r = ref[t]
        if r["flags"] & (O.TIE_EXPERT | O.TIE_GROUP):
            ties.append(t)
            continue
        assert within_tol(y[t], r["y"]), (t, float(np.max(np.abs(y[t] - r["y"]))))
    assert len(ties) < len(tokens)


def test_grouped_glm_decode_batch32(glm_g32):
    _check(glm_g32, synth.hidden_states(SH, 32, seed=0, step=1), [0, 31])


def test_grouped_glm_mtp_verify_192(glm_g32):
    _check(glm_g32, synth.mtp_hidden_states(SH, 64, 3, 0.8, seed=0, step=2), [0, 100, 191])


def test_grouped_glm_prefill_2048(glm_g32):
    _check(glm_g32, synth.hidden_states(SH, 2048, seed=0, step=3), [0, 2047])


def test_grouped_glm_paths_agree(glm_g32):
    x = synth.hidden_states(SH, 64, seed=0, step=4)
    y0 = _forward(glm_g32, x)
    assert np.array_equal(y0.view(np.uint32), _forward(glm_g32, x, gemm_min=1000).view(np.uint32))
    assert np.array_equal(y0.view(np.uint32), _forward(glm_g32, x, gemm_min=1).view(np.uint32))
