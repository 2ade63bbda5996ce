"""GPU parity over seeded random configurations: router shape (experts, groups,
kept groups, top-K), hidden and intermediate sizes, shared experts, batch size,
GEMV/MFMA threshold, weight width (int4 / int8), grouped int4 scales and
adaptive top-p, drawn together so that combinations the hand-picked cases do
not reach are exercised. Every tap of every token without a router near-tie is
compared bit for bit with the oracle; tokens with a near-tie are skipped (and
must be a minority).
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
N_CASES = 64


def _draw(i):
    """One configuration from a seeded generator (independent of the library)."""
    rng = np.random.default_rng(1000 + i)
    G = int(rng.choice([1, 2, 4, 8]))
    n = int(rng.choice([2, 3, 4, 8, 12, 16, 32]))
    E = G * n
    if E < 2:
        E, n = 2, 2
    KG = int(rng.integers(1, G + 1))
    K = int(rng.integers(1, min(32, KG * n) + 1))
    H = 64 * int(rng.integers(1, 9))
    I = 64 * int(rng.integers(1, 5))
    NS = int(rng.integers(0, 3))
    T = int(rng.choice([1, 3, 8, 17, 40, 70]))
    gemm_min = int(rng.choice([0, 1, 3, 1000]))
    wb = int(rng.choice([4, 4, 8]))
    gs = 0
    if wb == 4 and rng.random() < 0.4:
        cands = [g for g in (32, 64, 128) if H % g == 0 and I % g == 0]
        gs = int(rng.choice(cands))
    topp = float(rng.choice([0.0, 0.0, 0.5, 0.8]))
    sh = synth.Shape(H, E, G, KG, K, I, NS, float(rng.choice([1.0, 2.5])), bias_kind="uniform")
    return sh, T, gemm_min, wb, gs, topp, 500 + i


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_configuration(i):
    sh, T, gemm_min, wb, gs, topp, seed = _draw(i)
    layer = GpuLayer(sh, seed=seed, weight_bits=wb, group_size=gs)
    ref = oracle_layer(sh, seed=seed, weight_bits=wb, group_size=gs)
    x = synth.hidden_states(sh, T, seed=seed)
    H, I, K, NS = sh.hidden, sh.inter, sh.top_k, sh.n_shared
    R = T * K + NS * T
    cfg = config_of(sh, gemm_min, wb, gs, topp)
    bufs = dict(topk_ids=torch.empty((T, K), dtype=torch.int32, device=DEV),
                topk_w=torch.empty((T, K), dtype=torch.float32, device=DEV),
                near_tie=torch.empty(T, dtype=torch.uint8, device=DEV),
                qx=torch.empty((T, H), dtype=torch.int8, device=DEV),
                h=torch.zeros((R, I), dtype=torch.float32, device=DEV),
                qh=torch.zeros((R, I), dtype=torch.int8, device=DEV),
                e_out=torch.zeros((R, H), dtype=torch.float32, device=DEV))
    y = torch.empty((T, H), dtype=torch.float32, device=DEV)
    ws = torch.empty(moe.moe_workspace_bytes(cfg, T), dtype=torch.uint8, device=DEV)
    moe.moe_layer_forward(cfg, layer.weights(), torch.from_numpy(x).to(DEV), y, ws, moe.taps(-1, **bufs))
    torch.cuda.synchronize()
    g = {k: v.cpu().numpy() for k, v in bufs.items()}
    yg = y.cpu().numpy()
    yr, tr = O.layer_forward(O.Cfg.of(sh, group=gs, topp=topp), x, ref)
    assert np.array_equal(g["near_tie"], tr["flags"])
    clean = (tr["flags"] & (O.TIE_EXPERT | O.TIE_GROUP)) == 0
    assert clean.sum() > T // 2, (i, int(clean.sum()))
    assert np.array_equal(g["topk_ids"][clean], tr["ids"][clean])
    assert np.array_equal(g["topk_w"][clean].view(np.uint32), tr["w"][clean].view(np.uint32))
    assert np.array_equal(g["qx"], tr["qx"])
    # rows of the clean tokens' kept slots and their shared rows
    rows = [t * K + k for t in np.nonzero(clean)[0] for k in range(K) if tr["ids"][t, k] >= 0]
    rows += [T * K + s * T + t for s in range(NS) for t in np.nonzero(clean)[0]]
    rows = np.array(sorted(rows), dtype=np.int64)
    for k in ("h", "e_out"):
        assert np.array_equal(g[k][rows].view(np.uint32), tr[k][rows].view(np.uint32)), (i, k)
    assert np.array_equal(g["qh"][rows], tr["qh"][rows]), i
    assert np.array_equal(yg[clean].view(np.uint32), yr[clean].view(np.uint32)), i
