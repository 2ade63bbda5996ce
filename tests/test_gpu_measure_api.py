"""GPU tests of the measurement-only entry points: stage timing events
(moe_prof_*) and the memory microbenchmarks that calibrate the byte counters
(moe_membench_*), and the compute-rate kernels (moe_peakbench_*). Timing must
not change a forward's result; the stage mask selects the stages that are timed;
the read kernel folds every word it is given; the copy kernel copies every byte;
the compute-rate kernels run every step they count (their outputs equal the
closed forms of the work done).
"""
import numpy as np
import pytest

from synth import synth
from tests.harness import GpuLayer, config_of

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import int4_quantized_expert_amd as moe  # noqa: E402
from int4_quantized_expert_amd import _lib  # noqa: E402

DEV = torch.device("cuda:0")


def _forward(layer, cfg, x):
    T = x.shape[0]
    y = torch.empty((T, layer.shape.hidden), dtype=torch.float32, device=DEV)
    ws = torch.empty(moe.moe_workspace_bytes(cfg, T), dtype=torch.uint8, device=DEV)
    moe.moe_layer_forward(cfg, layer.weights(), x, y, ws)
    torch.cuda.synchronize()
    return y.cpu().numpy()


@pytest.mark.parametrize("gemm_min", [1000, 1])
def test_stage_timing_selected_stages_and_same_result(gemm_min):
    sh = synth.TINY
    layer = GpuLayer(sh)
    cfg = config_of(sh, gemm_min)
    x = torch.from_numpy(synth.hidden_states(sh, 16, seed=3)).to(DEV)
    y0 = _forward(layer, cfg, x)
    picked = ("router", "dispatch", "combine") + (("gateup_mfma",) if gemm_min == 1 else ("gateup_gemv",))
    moe.moe_prof_enable(3, picked)
    try:
        ys = [_forward(layer, cfg, x) for _ in range(3)]
        ms = moe.moe_prof_read(3)
    finally:
        moe.moe_prof_disable()
    for y in ys:
        assert np.array_equal(y.view(np.uint32), y0.view(np.uint32))
    assert ms.shape == (3, moe.MOE_N_STAGES)
    for s, name in enumerate(_lib.STAGES):
        if name in picked:
            assert np.all(np.isfinite(ms[:, s])) and np.all(ms[:, s] >= 0.0), name
        else:
            assert np.all(np.isnan(ms[:, s])), name


def test_stage_timing_rejects_bad_call_counts():
    for n in (0, 100001):
        with pytest.raises(moe.MoeError) as ei:
            moe.moe_prof_enable(n)
        assert ei.value.rc == moe.MOE_E_ARG


@pytest.mark.parametrize("nbytes,blocks", [(16, 1), (1 << 20, 7), ((1 << 20) + 48, 300)])
def test_membench_copy_copies_every_byte(nbytes, blocks):
    g = torch.Generator(device="cpu").manual_seed(nbytes)
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, generator=g).to(DEV)
    dst = torch.zeros(nbytes, dtype=torch.uint8, device=DEV)
    moe.moe_membench_copy(src, dst, blocks)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)


@pytest.mark.parametrize("unroll", [1, 2, 4, 8])
def test_membench_read_folds_every_word(unroll):
    # 3 blocks x 256 lanes over 2000 words: some lanes fold 3 words, some 2. Words are zero except those of
    # one lane, whose exclusive-or fold is planted to equal the value that makes the kernel write the sink.
    n16, lanes, lane = 2000, 3 * 256, 100
    words = np.zeros((n16, 4), np.uint32)
    mine = list(range(lane, n16, lanes))
    assert len(mine) == 3
    words[mine[0]] = [0x12345678, 0, 0, 0]
    words[mine[1]] = [0, 0x0F0F0F0F, 0, 0]
    words[mine[2]] = [0, 0, 0, 0x12345678 ^ 0x0F0F0F0F ^ 0x9E3779B9]
    buf = torch.from_numpy(words.view(np.uint8).reshape(-1).copy()).to(DEV)
    sink = torch.zeros(1, dtype=torch.int32, device=DEV)
    moe.moe_membench_read(buf, 3, unroll, sink)
    torch.cuda.synchronize()
    assert int(sink.cpu().numpy().view(np.uint32)[0]) == 0x9E3779B9
    # without the last planted word no lane's fold matches: the sink stays untouched
    words[mine[2]] = 0
    buf = torch.from_numpy(words.view(np.uint8).reshape(-1).copy()).to(DEV)
    sink.zero_()
    moe.moe_membench_read(buf, 3, unroll, sink)
    torch.cuda.synchronize()
    assert int(sink.cpu()[0]) == 0


def test_membench_rejects_bad_arguments():
    buf = torch.zeros(24, dtype=torch.uint8, device=DEV)  # not a whole number of 16-byte words
    sink = torch.zeros(1, dtype=torch.int32, device=DEV)
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_membench_read(buf, 1, 1, sink)
    assert ei.value.rc == moe.MOE_E_SHAPE
    buf = torch.zeros(32, dtype=torch.uint8, device=DEV)
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_membench_read(buf, 1, 3, sink)
    assert ei.value.rc == moe.MOE_E_ARG
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_membench_copy(buf, torch.zeros(32, dtype=torch.uint8, device=DEV), 0)
    assert ei.value.rc == moe.MOE_E_SHAPE


@pytest.mark.parametrize("blocks,iters,value", [(1, 1, 1), (3, 7, 3), (512, 100, -2), (64, 1000, 1)])
def test_peakbench_mfma_runs_every_step(blocks, iters, value):
    out = torch.full((blocks * 256,), -1, dtype=torch.int32, device=DEV)
    moe.moe_peakbench_mfma_i8(blocks, iters, value, out)
    torch.cuda.synchronize()
    # four chains of iters MFMAs, each adding 32 * value^2 to all 16 elements a lane holds
    assert bool((out == 2048 * value * value * iters).all())


@pytest.mark.parametrize("blocks,iters", [(1, 1), (5, 33), (512, 1000)])
def test_peakbench_valu_runs_every_step(blocks, iters):
    out = torch.full((blocks * 256,), -1.0, dtype=torch.float32, device=DEV)
    moe.moe_peakbench_valu_fma(blocks, iters, 1.0, 0.0, out)
    torch.cuda.synchronize()
    lane = torch.arange(blocks * 256, device=DEV) % 64
    assert bool((out == (8 * lane + 28).float()).all())
    if iters <= 100:  # a multiplier of one half: the result shows the run length (exact, no underflow)
        moe.moe_peakbench_valu_fma(blocks, iters, 0.5, 0.0, out)
        torch.cuda.synchronize()
        assert bool((out.double() == (8 * lane + 28).double() * (0.5 ** iters)).all())


def test_peakbench_rejects_bad_arguments():
    out = torch.empty(256, dtype=torch.int32, device=DEV)
    for blocks, iters in ((0, 1), (1, 0), (-1, 5)):
        assert _lib._lib.moe_peakbench_mfma_i8(blocks, iters, 1, _lib._ptr(out), None) == moe.MOE_E_SHAPE
        assert _lib._lib.moe_peakbench_valu_fma(blocks, iters, 1.0, 0.0, _lib._ptr(out), None) == moe.MOE_E_SHAPE
    assert _lib._lib.moe_peakbench_mfma_i8(1, 1, 1, None, None) == moe.MOE_E_NULL
