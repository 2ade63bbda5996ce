"""GPU parity for int8 expert weights (weight_bits = 8): per-row symmetric int8
codes with one fp32 scale per row, the precision the colibrì pages (Show HN,
implemented features) require of the MTP head, dotted against the same Q8_0
activations as the int4 experts.

The encoder is bit-exact against the oracle's; every tap of the tiny layer is
bit-exact on the GEMV path, the MFMA path and a mix; at the GLM-5.2 layer shape
sampled tokens are checked one at a time as for int4 (router bits exact, outputs
within |gpu - oracle| <= max(1e-5 |oracle|, 1e-6)).
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


@pytest.mark.parametrize("rows,cols", [(64, 32), (128, 256), (192, 96), (4096, 6144)])
def test_quantize_int8_bitexact(rows, cols):
    w = synth.normal(rows * cols, 1, 98, 0.02).reshape(rows, cols)
    w[3] = 0.0
    w[5, 7] = np.float32(0.5)  # one dominant element: the rest of the row rounds to small codes
    w[6, :4] = [0.5, -0.5, 0.25 + 1e-9, -0.5 * (0.5 / 127)]  # +-127 at the ends, a half-way code
    codes = torch.empty(rows * cols, dtype=torch.uint8, device=DEV)
    scales = torch.empty(rows, dtype=torch.float32, device=DEV)
    moe.moe_quantize_int8(_t(w), codes, scales)
    q_gpu = O.unpack_int8_tiled64(_np(codes), rows, cols)
    q_ref, s_ref = O.quant_int8_rows(w)
    assert np.array_equal(_np(scales).view(np.uint32), s_ref.view(np.uint32))
    assert np.array_equal(q_gpu, q_ref)
    assert q_gpu.min() >= -127


def test_quantize_int8_rejects_bad_shapes():
    w = torch.zeros((64, 48), dtype=torch.float32, device=DEV)
    codes = torch.empty(64 * 48, dtype=torch.uint8, device=DEV)
    scales = torch.empty(64, dtype=torch.float32, device=DEV)
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_quantize_int8(w, codes, scales)
    assert ei.value.rc == moe.MOE_E_SHAPE


# ------------------------------------------------------------------ tiny layer

@pytest.fixture(scope="module")
def tiny8():
    return GpuLayer(synth.TINY, weight_bits=8)


@pytest.fixture(scope="module")
def tiny8_ref():
    return oracle_layer(synth.TINY, weight_bits=8)


def _run(layer, x, gemm_min=0, sum_slot=-1, want_taps=True):
    sh = layer.shape
    H, I, K, E, NS = sh.hidden, sh.inter, sh.top_k, sh.n_experts, layer.NS
    cfg = config_of(sh, gemm_min, 8)
    T = x.shape[0]
    R = T * K + NS * T
    y = torch.empty((T, H), dtype=torch.float32, device=DEV)
    bufs = {}
    if want_taps:
        bufs = dict(topk_ids=torch.empty((T, K), dtype=torch.int32, device=DEV),
                    topk_w=torch.empty((T, K), dtype=torch.float32, device=DEV),
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


@pytest.mark.parametrize("T", [8, 16, 64])
@pytest.mark.parametrize("gemm_min", [1000, 1, 4])
def test_int8_layer_tiny_all_stages(tiny8, tiny8_ref, gemm_min, T):
    """Every tap bit-exact against the oracle with int8 experts: block sums of int8 x int8 are exact in int32
    (32 * 127 * 127 < 2^31), so the GEMV and MFMA paths give the oracle's bits."""
    sh = synth.TINY
    K = sh.top_k
    x = synth.hidden_states(sh, T, seed=21)
    slot = 3
    y, tp = _run(tiny8, x, gemm_min, sum_slot=slot)
    yr, tr = O.layer_forward(O.Cfg.of(sh), x, tiny8_ref)
    assert not (tr["flags"] & (O.TIE_EXPERT | O.TIE_GROUP)).any()
    assert np.array_equal(tp["topk_ids"], tr["ids"])
    assert np.array_equal(tp["qx"], tr["qx"]) and np.array_equal(tp["dx"], tr["dx"])
    assert np.array_equal(tp["h"].view(np.uint32), tr["h"].view(np.uint32))
    assert np.array_equal(tp["qh"], tr["qh"]) and np.array_equal(tp["dh"], tr["dh"])
    assert np.array_equal(tp["e_out"].view(np.uint32), tr["e_out"].view(np.uint32))
    assert np.array_equal(y.view(np.uint32), yr.view(np.uint32))
    e = tr["ids"].reshape(-1)[slot]
    q13, q2 = tiny8_ref.q13[e], tiny8_ref.q2[e]
    S13 = (q13.astype(np.int64) * tr["qx"][slot // K].astype(np.int64)[None]).reshape(2 * sh.inter, -1, 32).sum(2)
    S2 = (q2.astype(np.int64) * tr["qh"][slot].astype(np.int64)[None]).reshape(sh.hidden, -1, 32).sum(2)
    assert np.array_equal(tp["gateup_sums"], S13)
    assert np.array_equal(tp["down_sums"], S2)


@pytest.mark.parametrize("T", [1, 33, 77])
def test_int8_layer_tiny_ragged(tiny8, tiny8_ref, T):
    sh = synth.TINY
    x = synth.hidden_states(sh, T, seed=80 + T)
    y, tp = _run(tiny8, x, gemm_min=0)
    yr, tr = O.layer_forward(O.Cfg.of(sh), x, tiny8_ref)
    clean = (tr["flags"] & (O.TIE_EXPERT | O.TIE_GROUP)) == 0
    assert np.array_equal(tp["topk_ids"][clean], tr["ids"][clean])
    assert within_tol(y[clean], yr[clean])


def test_int8_differs_from_int4(tiny8):
    """The width is honoured: the same fp32 weights as int4 give a different (coarser) result."""
    sh = synth.TINY
    x = synth.hidden_states(sh, 8, seed=22)
    y8, _ = _run(tiny8, x, want_taps=False)
    l4 = GpuLayer(sh)
    cfg4 = config_of(sh, 0, 4)
    y4 = torch.empty((8, sh.hidden), dtype=torch.float32, device=DEV)
    ws = torch.empty(moe.moe_workspace_bytes(cfg4, 8), dtype=torch.uint8, device=DEV)
    moe.moe_layer_forward(cfg4, l4.weights(), _t(x), y4, ws)
    assert not np.array_equal(_np(y4), y8)


def test_rejects_bad_weight_bits(tiny8):
    sh = synth.TINY
    x = torch.zeros((4, sh.hidden), dtype=torch.float32, device=DEV)
    y = torch.empty_like(x)
    for wb in (2, 5, 16):
        cfg = config_of(sh, 0, wb)
        assert moe.moe_workspace_bytes(cfg, 4) == 0
        ws = torch.empty(1 << 20, dtype=torch.uint8, device=DEV)
        with pytest.raises(moe.MoeError) as ei:
            moe.moe_layer_forward(cfg, tiny8.weights(), x, y, ws)
        assert ei.value.rc == moe.MOE_E_ARG


# ------------------------------------------------------------------ GLM-5.2 layer shape

SH = synth.GLM


@pytest.fixture(scope="module")
def glm8():
    return GpuLayer(SH, weight_bits=8)


def _forward(layer, x, gemm_min=0):
    cfg = config_of(SH, gemm_min, 8)
    T = x.shape[0]
    xd = _t(x)
    ws = torch.empty(moe.moe_workspace_bytes(cfg, T), dtype=torch.uint8, device=DEV)
    y = torch.empty((T, SH.hidden), dtype=torch.float32, device=DEV)
    moe.moe_layer_forward(cfg, layer.weights(), xd, y, ws)
    return _np(y)


def _check(layer, x, tokens, gemm_min=0):
    y = _forward(layer, x, gemm_min)
    ref = oracle_tokens(SH, x, tokens, weight_bits=8)
    ties = []
    for t in tokens:
        r = ref[t]
        if r["flags"] & (O.TIE_EXPERT | O.TIE_GROUP):
            ties.append(t)
            continue
        assert within_tol(y[t], r["y"]), (t, float(np.max(np.abs(y[t] - r["y"]))))
    assert len(ties) < len(tokens)
    return y


def test_int8_glm_decode_batch32(glm8):
    _check(glm8, synth.hidden_states(SH, 32, seed=0, step=1), [0, 31])


def test_int8_glm_mtp_verify_192(glm8):
    _check(glm8, synth.mtp_hidden_states(SH, 64, 3, 0.8, seed=0, step=2), [0, 100, 191])


def test_int8_glm_paths_agree(glm8):
    x = synth.hidden_states(SH, 64, seed=0, step=4)
    y0 = _forward(glm8, x)
    assert np.array_equal(y0.view(np.uint32), _forward(glm8, x, gemm_min=1000).view(np.uint32))
    assert np.array_equal(y0.view(np.uint32), _forward(glm8, x, gemm_min=1).view(np.uint32))
