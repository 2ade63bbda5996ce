"""One tiny MoE-layer forward on cuda:0 through the C ABI, checked against the oracle."""
from __future__ import annotations

import numpy as np


def run_smoke() -> None:
    import torch

    import int4_quantized_expert_amd as moe
    from oracle import oracle as O
    from synth import synth
    from tests.harness import GpuLayer, config_of, oracle_layer, within_tol

    if not torch.cuda.is_available():
        raise RuntimeError("smoke needs a GPU (cuda:0)")
    dev = torch.device("cuda:0")
    sh = synth.TINY
    T = 8
    layer = GpuLayer(sh, device="cuda:0")
    x = synth.hidden_states(sh, T)
    cfg = config_of(sh)
    ws = torch.empty(moe.moe_workspace_bytes(cfg, T), dtype=torch.uint8, device=dev)
    y = torch.empty((T, sh.hidden), dtype=torch.float32, device=dev)
    moe.moe_layer_forward(cfg, layer.weights(), torch.from_numpy(x).to(dev), y, ws)
    torch.cuda.synchronize()
    yr, tr = O.layer_forward(O.Cfg.of(sh), x, oracle_layer(sh))
    yg = y.cpu().numpy()
    if not within_tol(yg, yr):
        raise AssertionError(f"smoke: layer output differs from the oracle (max abs {np.abs(yg - yr).max():.3e})")
    print(f"smoke ok: tiny MoE layer T={T}, max |gpu-oracle| = {np.abs(yg - yr).max():.3e}")


if __name__ == "__main__":
    run_smoke()
