"""GPU checks of the converters from the canonical packing of the pages' weight
formats ("Show HN: 느린 컴퓨터에서 GLM 5.2 실행하기", implemented features: packed
int4 and int8 weights with per-row scales) into the library's row-tiled layouts.

The canonical bytes are written by the oracle's own packer (row-major, element 2j
in the low nibble of byte j); the tiled bytes are read back by the oracle's
layout readers. A converter is a byte permutation, so everything is compared bit
for bit: codes read back through the oracle equal the codes packed, and the
converted bytes equal what the fp32 encoders (moe_quantize_*) write for the same
weights, which makes a layer built from canonical codes the same layer.
"""
import numpy as np
import pytest

from oracle import oracle as O
from synth import synth

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


SHAPES = [(64, 32), (128, 256), (192, 96), (4096, 6144), (6144, 2048)]


@pytest.mark.parametrize("rows,cols", SHAPES)
def test_tile_int4_reads_back(rows, cols):
    rng = np.random.default_rng(rows * 7 + cols)
    q = rng.integers(-8, 8, size=(rows, cols), dtype=np.int8)  # every nibble value, -8 included
    canon = O.pack_int4(q)
    tiled = torch.full((rows * cols // 2,), 0xAB, dtype=torch.uint8, device=DEV)
    moe.moe_tile_int4(_t(canon.reshape(rows, cols // 2)), tiled)
    assert np.array_equal(O.unpack_int4_tiled64(_np(tiled), rows, cols), q)


@pytest.mark.parametrize("rows,cols", SHAPES)
def test_tile_int4_equals_encoder(rows, cols):
    w = synth.normal(rows * cols, 1, 211, 0.02).reshape(rows, cols)
    w[1] = 0.0
    q, s = O.quant_int4_rows(w)
    tiled = torch.empty(rows * cols // 2, dtype=torch.uint8, device=DEV)
    moe.moe_tile_int4(_t(O.pack_int4(q).reshape(rows, cols // 2)), tiled)
    enc = torch.empty(rows * cols // 2, dtype=torch.uint8, device=DEV)
    enc_s = torch.empty(rows, dtype=torch.float32, device=DEV)
    moe.moe_quantize_int4(_t(w), enc, enc_s)
    assert np.array_equal(_np(tiled), _np(enc))
    assert np.array_equal(_np(enc_s).view(np.uint32), s.view(np.uint32))  # row scales: same layout on both sides


@pytest.mark.parametrize("rows,cols", SHAPES)
def test_tile_int8_reads_back_and_equals_encoder(rows, cols):
    rng = np.random.default_rng(rows * 5 + cols)
    q = rng.integers(-128, 128, size=(rows, cols), dtype=np.int8)
    tiled = torch.full((rows * cols,), 0xAB, dtype=torch.uint8, device=DEV)
    moe.moe_tile_int8(_t(q), tiled)
    assert np.array_equal(O.unpack_int8_tiled64(_np(tiled), rows, cols), q)
    w = synth.normal(rows * cols, 1, 212, 0.02).reshape(rows, cols)
    q8, _ = O.quant_int8_rows(w)
    moe.moe_tile_int8(_t(q8), tiled)
    enc = torch.empty(rows * cols, dtype=torch.uint8, device=DEV)
    enc_s = torch.empty(rows, dtype=torch.float32, device=DEV)
    moe.moe_quantize_int8(_t(w), enc, enc_s)
    assert np.array_equal(_np(tiled), _np(enc))


@pytest.mark.parametrize("rows,cols,group", [(64, 64, 32), (128, 256, 64), (4096, 6144, 128), (6144, 2048, 32)])
def test_tile_grouped_equals_encoder(rows, cols, group):
    w = synth.normal(rows * cols, 1, 213, 0.02).reshape(rows, cols)
    q, s = O.quant_int4_grouped(w, group)
    ng = cols // group
    codes = torch.empty(rows * cols // 2, dtype=torch.uint8, device=DEV)
    moe.moe_tile_int4(_t(O.pack_int4(q).reshape(rows, cols // 2)), codes)
    sc = torch.empty(rows * ng, dtype=torch.float32, device=DEV)
    moe.moe_tile_group_scales(_t(s), sc)
    assert np.array_equal(O.unpack_scales_tiled64(_np(sc), rows, ng).view(np.uint32), s.view(np.uint32))
    enc = torch.empty(rows * cols // 2, dtype=torch.uint8, device=DEV)
    enc_s = torch.empty(rows * ng, dtype=torch.float32, device=DEV)
    moe.moe_quantize_int4_grouped(_t(w), group, enc, enc_s)
    assert np.array_equal(_np(codes), _np(enc))
    assert np.array_equal(_np(sc).view(np.uint32), _np(enc_s).view(np.uint32))


def test_tile_rejects_bad_arguments():
    src = torch.zeros((64, 24), dtype=torch.uint8, device=DEV)  # 48 columns: not whole 32-element blocks
    dst = torch.zeros(64 * 48, dtype=torch.uint8, device=DEV)
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_tile_int4(src, dst)
    assert ei.value.rc == moe.MOE_E_SHAPE
    flat = torch.zeros(64 * 16 + 16, dtype=torch.uint8, device=DEV)
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_tile_int4(flat[1:1 + 64 * 16].view(64, 16), dst)  # a source that is not 16-byte aligned
    assert ei.value.rc == moe.MOE_E_ARG
    with pytest.raises(moe.ArgError):
        moe.moe_tile_int4(torch.zeros((128, 16), dtype=torch.uint8, device=DEV), dst[:1024])  # 2 KB into 1 KB
