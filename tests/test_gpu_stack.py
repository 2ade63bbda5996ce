"""Two GLM-5.2-shaped layers stacked with a residual stream: layer 0 resident in HBM, layer 1 with its routed
experts in pinned host memory behind a 64-slot LRU expert cache ("Show HN: 느린 컴퓨터에서 GLM 5.2 실행하기",
disk-streaming MoE and learning cache; "Colibri: 25GB RAM을 탑재한 노트북에서 744B AI 모델 실행하기", the
router's decisions and outputs do not depend on the tier holding an expert).

Residual chain (the stacked-decode reading): h0 = x; layer input = weightless RMSNorm(h) (eps 1e-6, fp32);
h1 = h0 + y0. The glue between layers runs in torch; it is not part of the MoE layer. Per step:
  - the streamed layer's output equals the same layer's all-resident forward bit for bit;
  - teacher-forced oracle parity on the streamed layer: the oracle gets the GPU's layer-1 input and must
    agree on router ids and weights (bit-exact, near-ties reported) and on y of sampled tokens within
    |gpu - oracle| <= max(1e-5 |oracle|, 1e-6);
  - hits + misses = unique experts, and a step after the first finds some experts resident.
"""
import numpy as np
import pytest

from oracle import oracle as O
from synth import synth
from tests import harness as HN
from tests.harness import GpuLayer, config_of, host_experts, oracle_router_all, oracle_slots, within_tol

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import int4_quantized_expert_amd as moe  # noqa: E402

DEV = torch.device("cuda:0")
SH = synth.GLM


def _rmsnorm(h):
    return h * torch.rsqrt(torch.mean(h * h, dim=1, keepdim=True) + 1e-6)


def test_two_layer_stack_streamed_layer_against_oracle():
    old = HN.ORACLE_CACHE_MAX
    HN.ORACLE_CACHE_MAX = 300
    try:
        _run()
    finally:
        HN._ORACLE_CACHE.clear()
        HN.ORACLE_CACHE_MAX = old


def _run():
    T, K, H, NS, E = 32, SH.top_k, SH.hidden, SH.n_shared, SH.n_experts
    cfg = config_of(SH)
    l0 = GpuLayer(SH, layer=0)
    l1 = GpuLayer(SH, layer=1)
    hx1, keep = host_experts(l1)
    cache = moe.ExpertCache(cfg, 64, T)
    ws = torch.empty(moe.moe_workspace_bytes(cfg, T), dtype=torch.uint8, device=DEV)
    compute, copy = torch.cuda.Stream(), torch.cuda.Stream()
    sample = [0, 9, 17, 31]
    prev = cache.stats()
    for step in range(3):
        print(f"stack step {step}", flush=True)
        x = torch.from_numpy(synth.hidden_states(SH, T, seed=0, step=40 + step)).to(DEV)
        y0 = torch.empty((T, H), dtype=torch.float32, device=DEV)
        moe.moe_layer_forward(cfg, l0.weights(), _rmsnorm(x).contiguous(), y0, ws)
        in1 = _rmsnorm(x + y0).contiguous()
        y1 = torch.empty((T, H), dtype=torch.float32, device=DEV)
        ids1 = torch.empty((T, K), dtype=torch.int32, device=DEV)
        w1 = torch.empty((T, K), dtype=torch.float32, device=DEV)
        tie1 = torch.empty(T, dtype=torch.uint8, device=DEV)
        torch.cuda.synchronize()
        cache.forward(l1.weights(), hx1, in1, y1, ws, compute, copy)
        torch.cuda.synchronize()
        # tier invariance: the streamed layer equals the resident one
        y_res = torch.empty((T, H), dtype=torch.float32, device=DEV)
        moe.moe_layer_forward(cfg, l1.weights(), in1, y_res, ws, moe.taps(topk_ids=ids1, topk_w=w1, near_tie=tie1))
        torch.cuda.synchronize()
        y1h, in1h = y1.cpu().numpy(), in1.cpu().numpy()
        assert np.array_equal(y1h.view(np.uint32), y_res.cpu().numpy().view(np.uint32)), step
        # teacher-forced oracle parity of the streamed layer on the GPU's layer input
        r = oracle_router_all(SH, in1h, layer=1)
        ids, w, fl = ids1.cpu().numpy(), w1.cpu().numpy(), tie1.cpu().numpy()
        assert np.array_equal(fl, r["flags"])
        clean = [t for t in range(T) if not r["flags"][t] & (O.TIE_EXPERT | O.TIE_GROUP)]
        assert len(clean) > T // 2
        for t in clean:
            assert np.array_equal(ids[t], r["ids"][t]), t
            if not r["zb"][t, ids[t]].any():
                assert np.array_equal(w[t].view(np.uint32), r["w"][t].view(np.uint32)), t
        pairs = [(t, int(ids[t, k]), False) for t in sample for k in range(K)] + \
                [(t, s, True) for t in sample for s in range(NS)]
        ref = oracle_slots(SH, in1h, pairs, layer=1)
        rows = {(t, e, sh): rr["out"] for (t, e, sh), rr in zip(pairs, ref)}
        for t in sample:
            er = np.stack([rows[(t, int(ids[t, k]), False)] for k in range(K)])[None]
            es = np.stack([rows[(t, s, True)] for s in range(NS)])[:, None]
            yref = O.combine(er, es, w[t:t + 1], ids[t:t + 1])[0]
            assert within_tol(y1h[t], yref), (step, t, float(np.max(np.abs(y1h[t] - yref))))
        st = cache.stats()
        u = len(np.unique(ids))
        assert (st["hits"] - prev["hits"]) + (st["misses"] - prev["misses"]) == u, step
        if step > 0:
            assert st["hits"] > prev["hits"], step
        prev = st
    cache.destroy()
    del keep
