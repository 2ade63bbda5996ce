"""GPU parity for the 64-position MFMA tiles (batches of 256 tokens and more):
both prefetch depths of their block ring (4 blocks when the block count is a
multiple of 4, 2 otherwise) for gate/up and down, with int4 row scales, int4
grouped scales and int8 weights, up to batches whose dispatch reads the ids
from global memory; and the 32-position tiles of small batches (T*K <= 512),
which run four tiles per workgroup, on shapes whose row-block counts are not
multiples of four (5 or 6 down tiles, 6 gate/up row blocks), so that some
wavefronts of the last workgroup have no tile. Every tap of every token
without a router near-tie is compared bit for bit with the oracle.
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

# hidden / 32 and inter / 32 blocks: 8 and 4 (ring of 4), 10 and 6 (ring of 2), 12 and 6 (4 for gate/up, 2 for down)
SHAPES = {
    "ring4": synth.Shape(256, 16, 4, 2, 4, 128, 1, 2.5, bias_kind="uniform"),
    "ring2": synth.Shape(320, 16, 4, 2, 4, 192, 1, 2.5, bias_kind="uniform"),
    "mixed": synth.Shape(384, 16, 4, 2, 4, 192, 2, 2.5, bias_kind="uniform"),
}


# Every shape and weight format at T = 300 (all MFMA) and 257 (mixed); large batches for one int4 and one int8
# shape: T = 3200 with top-4 is 12,800 slots, T = 6200 is 24,800, past the 24,576 up to which dispatch keeps
# the ids in LDS, so it reads them from global memory.
CASES = [(n, wb, gs, T, gm) for n in SHAPES for (wb, gs) in ((4, 0), (4, 64), (8, 0)) for (T, gm) in ((300, 1), (257, 70))]
CASES += [(n, wb, 0, T, gm) for (n, wb) in (("ring4", 4), ("mixed", 8)) for (T, gm) in ((3200, 1), (6200, 5))]
# small batches: all buckets (gemm_min 1) or those of 3+ tokens on the grouped 32-position tiles
CASES += [(n, wb, gs, 40, gm) for n in ("ring2", "mixed") for (wb, gs) in ((4, 0), (4, 64), (8, 0)) for gm in (1, 3)]


@pytest.mark.parametrize("name,wb,gs,T,gemm_min", CASES)
def test_wide_tiles_all_taps_bitexact(name, wb, gs, T, gemm_min):
    sh = SHAPES[name]
    seed = 70 + T
    layer = GpuLayer(sh, seed=seed, weight_bits=wb, group_size=gs)
    ref = oracle_layer(sh, seed=seed, weight_bits=wb, group_size=gs)
    x = synth.hidden_states(sh, T, seed=seed)
    H, I, K, NS = sh.hidden, sh.inter, sh.top_k, sh.n_shared
    R = T * K + NS * T
    cfg = config_of(sh, gemm_min, wb, gs)
    bufs = dict(topk_ids=torch.empty((T, K), dtype=torch.int32, device=DEV),
                near_tie=torch.empty(T, dtype=torch.uint8, device=DEV),
                h=torch.zeros((R, I), dtype=torch.float32, device=DEV),
                qh=torch.zeros((R, I), dtype=torch.int8, device=DEV),
                e_out=torch.zeros((R, H), dtype=torch.float32, device=DEV))
    y = torch.empty((T, H), dtype=torch.float32, device=DEV)
    ws = torch.empty(moe.moe_workspace_bytes(cfg, T), dtype=torch.uint8, device=DEV)
    moe.moe_layer_forward(cfg, layer.weights(), torch.from_numpy(x).to(DEV), y, ws, moe.taps(-1, **bufs))
    torch.cuda.synchronize()
    g = {k: v.cpu().numpy() for k, v in bufs.items()}
    yg = y.cpu().numpy()
    yr, tr = O.layer_forward(O.Cfg.of(sh, group=gs), x, ref)
    assert np.array_equal(g["near_tie"], tr["flags"])
    clean = (tr["flags"] & (O.TIE_EXPERT | O.TIE_GROUP)) == 0
    assert clean.sum() > 0.9 * T
    assert np.array_equal(g["topk_ids"][clean], tr["ids"][clean])
    toks = np.nonzero(clean)[0]
    rows = np.array(sorted([t * K + k for t in toks for k in range(K)] + [T * K + s * T + t for s in range(NS)
                                                                        for t in toks]), dtype=np.int64)
    for k in ("h", "e_out"):
        assert np.array_equal(g[k][rows].view(np.uint32), tr[k][rows].view(np.uint32)), k
    assert np.array_equal(g["qh"][rows], tr["qh"][rows])
    assert np.array_equal(yg[clean].view(np.uint32), yr[clean].view(np.uint32))
