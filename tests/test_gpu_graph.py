"""A layer forward captured as a HIP graph (the way a serving loop replays a decode step) gives the same bits as
the eager call on every replay, with eager forwards of other inputs and synchronisations between the replays.
The capture holds the library's launches on the caller's stream and the helper stream's fork and join."""
import numpy as np
import pytest

from synth import synth
from tests.harness import GpuLayer, config_of

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import int4_quantized_expert_amd as moe  # noqa: E402

DEV = torch.device("cuda:0")


@pytest.mark.parametrize("shape_name,T", [("TINY", 8), ("TINY", 64), ("GLM", 1), ("GLM", 32), ("GLM", 192)])
def test_graph_replay_equals_eager(shape_name, T):
    sh = getattr(synth, shape_name)
    layer = GpuLayer(sh)
    cfg = config_of(sh)
    w = layer.weights()
    x = torch.from_numpy(synth.hidden_states(sh, T, seed=0, step=60)).to(DEV)
    x2 = torch.from_numpy(synth.hidden_states(sh, T, seed=0, step=61)).to(DEV)
    ws = torch.empty(moe.moe_workspace_bytes(cfg, T), dtype=torch.uint8, device=DEV)
    y_ref = torch.empty((T, sh.hidden), dtype=torch.float32, device=DEV)
    moe.moe_layer_forward(cfg, w, x, y_ref, ws)
    torch.cuda.synchronize()
    ref = y_ref.cpu().numpy()
    cap = torch.cuda.Stream()
    y = torch.full((T, sh.hidden), float("nan"), dtype=torch.float32, device=DEV)
    with torch.cuda.stream(cap):
        moe.moe_layer_forward(cfg, w, x, y, ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        moe.moe_layer_forward(cfg, w, x, y, ws)
    ws2 = torch.empty_like(ws)
    y2 = torch.empty_like(y)
    for rep in range(4):
        y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(y.cpu().numpy().view(np.uint32), ref.view(np.uint32)), (shape_name, T, rep)
        # eager work between replays, on the same workspace and on another one
        moe.moe_layer_forward(cfg, w, x2, y2, ws if rep % 2 else ws2)
        torch.cuda.synchronize()
    del g
