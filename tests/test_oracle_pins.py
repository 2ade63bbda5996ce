"""Pins for the C oracle: each check compares it with something other than itself
(hand-derived goldens, closed forms, brute force, library routines, error bounds)."""
import itertools
import json
import math
import os
from collections import OrderedDict

import numpy as np
import pytest
import scipy.special

from oracle import oracle as O
from synth import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")
HW = json.load(open(os.path.join(GOLD, "hand_worked.json")))
U = 2.0 ** -24  # fp32 unit roundoff


def gamma(n):
    return n * U / (1 - n * U)


# ------------------------------------------------------------------ encodings

def test_int4_pack_roundtrip_all_bytes():
    allb = np.arange(256, dtype=np.uint8)
    q = O.unpack_int4(allb, 512)
    assert q.min() == -8 and q.max() == 7
    # low nibble first, two's complement: byte 0x8F -> (-1, -8)
    assert tuple(q[2 * 0x8F:2 * 0x8F + 2]) == (-1, -8)
    assert tuple(q[2 * 0x70:2 * 0x70 + 2]) == (0, 7)
    assert np.array_equal(O.pack_int4(q), allb)
    nib = np.array([a for a in range(-8, 8) for _ in (0, 1)], np.int8)
    assert np.array_equal(O.unpack_int4(O.pack_int4(nib), nib.size), nib)


def test_int4_tiled64_single_tile_is_rowmajor_and_bijective():
    rng = np.random.default_rng(1)
    q = rng.integers(-8, 8, size=(64, 32), dtype=np.int8)
    # one tile, one block: the layout degenerates to 64 consecutive 16-byte rows
    packed = O.pack_int4(q)
    assert np.array_equal(O.unpack_int4_tiled64(packed, 64, 32), q)
    # larger: every byte of the buffer is read exactly once (bijection)
    rows, cols = 128, 96
    buf = np.arange(rows * cols // 2, dtype=np.int64)
    seen = np.zeros(buf.size, np.int64)
    for r in range(rows):
        for b in range(cols // 32):
            base = ((r // 64) * (cols // 32) + b) * 1024 + (r % 64) * 16
            seen[base:base + 16] += 1
    assert np.all(seen == 1)
    q2 = rng.integers(-8, 8, size=(rows, cols), dtype=np.int8)
    dev = np.empty(rows * cols // 2, np.uint8)
    for r in range(rows):
        for b in range(cols // 32):
            base = ((r // 64) * (cols // 32) + b) * 1024 + (r % 64) * 16
            dev[base:base + 16] = O.pack_int4(q2[r, b * 32:(b + 1) * 32])
    assert np.array_equal(O.unpack_int4_tiled64(dev, rows, cols), q2)


def test_int4_quant_golden_and_bounds():
    g = HW["int4_halfway"]
    row = np.zeros((1, 32), np.float32)
    row[0, :len(g["row_head"])] = g["row_head"]
    q, s = O.quant_int4_rows(row)
    assert s[0] == g["expected_s"]
    assert list(q[0, :len(g["expected_q_head"])]) == g["expected_q_head"]
    w = synth.normal(64 * 256, 3, 77, 0.02).reshape(64, 256)
    w[5] = 0.0
    q, s = O.quant_int4_rows(w)
    assert s[5] == 0 and not q[5].any()
    assert np.abs(q).max() <= 7
    amax = np.abs(w).max(1)
    am = np.argmax(np.abs(w), 1)
    for r in range(64):
        if r == 5:
            continue
        assert abs(int(q[r, am[r]])) == 7
        err = np.abs(w[r].astype(np.float64) - s[r] * q[r].astype(np.float64))
        assert err.max() <= s[r] / 2 * (1 + 1e-6) + 1e-12
        assert abs(s[r] - amax[r] / 7) <= 2 * U * amax[r] / 7
    # exact multiples reproduce their integers
    k = np.array([[7, -7, 3, 0, -2, 1] + [0] * 26], np.float32)
    q, s = O.quant_int4_rows(k * np.float32(0.25))
    assert s[0] == 0.25 and np.array_equal(q[0], k[0].astype(np.int8))


def test_int8_quant_golden_and_bounds():
    g = HW["int8_halfway"]
    row = np.zeros((1, 32), np.float32)
    row[0, :len(g["row_head"])] = g["row_head"]
    q, s = O.quant_int8_rows(row)
    assert s[0] == g["expected_s"]
    assert list(q[0, :len(g["expected_q_head"])]) == g["expected_q_head"]
    w = synth.normal(64 * 256, 3, 78, 0.02).reshape(64, 256)
    w[9] = 0.0
    q, s = O.quant_int8_rows(w)
    assert s[9] == 0 and not q[9].any()
    assert np.abs(q.astype(np.int32)).max() <= 127
    amax = np.abs(w).max(1)
    am = np.argmax(np.abs(w), 1)
    for r in range(64):
        if r == 9:
            continue
        assert abs(int(q[r, am[r]])) == 127
        err = np.abs(w[r].astype(np.float64) - s[r] * q[r].astype(np.float64))
        assert err.max() <= s[r] / 2 * (1 + 1e-6) + 1e-12
        assert abs(s[r] - amax[r] / 127) <= 2 * U * amax[r] / 127


def test_int8_tiled64_layout_against_its_formula():
    """A plain packer written from the documented address formula, then the oracle's reader."""
    rng = np.random.default_rng(31)
    rows, cols = 128, 96
    q = rng.integers(-127, 128, size=(rows, cols)).astype(np.int8)
    buf = np.zeros(rows * cols, np.uint8)
    nb = cols // 32
    for r in range(rows):
        for b in range(nb):
            base = ((r // 64) * nb + b) * 2048 + (r % 64) * 32
            for e in range(32):
                g, m = divmod(e, 8)
                pos = 8 * g + (m // 2 if m % 2 == 0 else 4 + m // 2)
                buf[base + pos] = np.uint8(int(q[r, b * 32 + e]) & 0xFF)
    assert np.array_equal(O.unpack_int8_tiled64(buf, rows, cols), q)


def test_int4_grouped_golden():
    g = HW["int4_grouped_hand"]
    row = np.zeros((1, g["cols"]), np.float32)
    for k, v in g["nonzero"].items():
        row[0, int(k)] = v
    q, s = O.quant_int4_grouped(row, g["group"])
    assert s.shape == (1, g["cols"] // g["group"])
    assert np.array_equal(s[0], np.array(g["expected_s"], np.float32))
    want = np.zeros(g["cols"], np.int8)
    for k, v in g["expected_q"].items():
        want[int(k)] = v
    assert np.array_equal(q[0], want)


def test_int4_grouped_whole_row_group_is_per_row():
    """One group spanning the row is exactly the per-row quantizer."""
    w = synth.normal(64 * 256, 5, 61, 0.02).reshape(64, 256)
    w[7] = 0.0
    q, s = O.quant_int4_grouped(w, 256)
    qr, sr = O.quant_int4_rows(w)
    assert np.array_equal(q, qr) and np.array_equal(s[:, 0].view(np.uint32), sr.view(np.uint32))


@pytest.mark.parametrize("group", [32, 64, 128])
def test_int4_grouped_bounds(group):
    """Every group reaches +-7 at its largest element, codes stay in [-7, 7], and the reconstruction error of
    each element is at most half its group's step."""
    w = synth.normal(64 * 512, 6, 62, 0.02).reshape(64, 512)
    w[3, :group] = 0.0  # one all-zero group
    q, s = O.quant_int4_grouped(w, group)
    assert q.min() >= -7 and q.max() <= 7
    ng = 512 // group
    sg = np.repeat(s, group, axis=1).astype(np.float64)
    err = np.abs(w.astype(np.float64) - sg * q)
    assert np.all(err <= sg / 2 * (1 + 4 * U) + 1e-30)
    amax = np.abs(w.reshape(64, ng, group)).max(2)
    assert np.all(s == (amax / np.float32(7.0)).astype(np.float32))
    big = np.abs(q.reshape(64, ng, group)).max(2)
    assert np.all(big[amax > 0] == 7) and np.all(big[amax == 0] == 0)
    # finer groups never lose to one scale per row on the row's worst element
    _, sr = O.quant_int4_rows(w)
    assert np.all(err.max(1) <= sr.astype(np.float64) / 2 * (1 + 4 * U))


def test_scales_tiled64_golden():
    g = HW["scales_tiled64"]
    rows, ng = g["rows"], g["ng"]
    buf = np.arange(rows * ng, dtype=np.float32)
    sc = O.unpack_scales_tiled64(buf, rows, ng)
    for r, gi, idx in g["points"]:
        assert sc[r, gi] == idx
    assert np.array_equal(np.sort(sc.ravel()), buf)  # a bijection


def test_q8_0_golden_and_bounds():
    g = HW["q8_0_halfway"]
    blk = np.zeros(64, np.float32)
    blk[:len(g["block_head"])] = g["block_head"]
    q, d = O.q8_0(blk)
    assert d[0] == g["expected_d"] and d[1] == 0.0
    assert list(q[:len(g["expected_q_head"])]) == g["expected_q_head"]
    assert not q[32:].any()
    x = synth.normal(32 * 4096, 0, 5, 1.0)
    q, d = O.q8_0(x)
    xb = x.reshape(-1, 32).astype(np.float64)
    qb = q.reshape(-1, 32).astype(np.float64)
    err = np.abs(xb - d[:, None].astype(np.float64) * qb)
    assert np.all(err <= d[:, None] / 2 * (1 + 2.0 ** -22) + 1e-30)
    am = np.argmax(np.abs(xb), 1)
    assert np.all(np.abs(qb[np.arange(qb.shape[0]), am]) == 127)
    # disagreement count with an fp64 round(x/d) definition is tiny
    ref = np.clip(np.sign(xb) * np.floor(np.abs(xb) / d[:, None].astype(np.float64) + 0.5), -127, 127)
    assert (ref != qb).sum() <= 4
    k = np.arange(-16, 16, dtype=np.float32)
    k[0] = -127
    q, d = O.q8_0(k * np.float32(0.5))
    assert d[0] == 0.5 and np.array_equal(q, k.astype(np.int8))


# ------------------------------------------------------------------- router

def test_router_logits_vs_exact_sum():
    x = synth.normal(5 * 384, 0, 11, 1.0).reshape(5, 384)
    W = synth.normal(24 * 384, 0, 12, 0.02).reshape(24, 384)
    z = O.router_logits(x, W)
    exact = np.empty_like(z)
    for t in range(5):
        for e in range(24):
            exact[t, e] = np.float32(math.fsum((x[t].astype(np.float64) * W[e].astype(np.float64)).tolist()))
    # fp64 sequential vs correctly rounded sum agree after rounding to fp32 (an ulp apart at most)
    ulp = np.spacing(np.abs(exact))
    assert np.all(np.abs(z - exact) <= ulp)
    assert (z == exact).mean() >= 0.99
    # transposed operand would be a different shape entirely; a swapped index changes values
    assert not np.allclose(O.router_logits(x, W[::-1]), z)


def _route_one(E, G, KG, K, rsf, z, bias):
    cfg = O.Cfg(32, E, G, KG, K, 32, 0, rsf)
    return O.route(cfg, np.asarray(z, np.float32)[None], np.asarray(bias, np.float32), want_scores=True)


@pytest.mark.parametrize("case", ["router_group_tie", "router_clear", "router_expert_tie"])
def test_route_golden(case):
    g = HW[case]
    ids, w, fl, s, c = _route_one(g["E"], g["G"], g["topk_group"], g["K"], g["rsf"], g["z"], g["bias"])
    assert list(ids[0]) == g["expected_ids"]
    assert list(w[0]) == g["expected_w"]
    assert int(fl[0]) == g["expected_flags"]


def test_sigmoid_vs_library_and_symmetry():
    z = synth.normal(4 * 64, 0, 13, 3.0).reshape(4, 64)
    z[0, 0] = 0.0
    cfg = O.Cfg(32, 64, 8, 8, 8, 32, 0, 1.0)
    _, _, _, s, c = O.route(cfg, z, np.zeros(64, np.float32), want_scores=True)
    ref = scipy.special.expit(z.astype(np.float64)).astype(np.float32)
    assert np.all(np.abs(s - ref) <= np.spacing(ref))
    assert (s == ref).mean() > 0.99
    assert s[0, 0] == 0.5
    _, _, _, s2, _ = O.route(cfg, -z, np.zeros(64, np.float32), want_scores=True)
    assert np.all(np.abs((s + s2).astype(np.float64) - 1.0) <= 2 * np.spacing(np.float32(1.0)))
    assert np.array_equal(c, s)  # zero bias


def _brute_route(cE, G, KG, K):
    n = cE.size // G
    gs = np.array([np.float32(np.sort(cE[g * n:(g + 1) * n])[-1]) + np.float32(np.sort(cE[g * n:(g + 1) * n])[-2])
                   for g in range(G)], np.float32)
    best = max(itertools.combinations(range(G), KG),
               key=lambda gset: (sum(float(gs[g]) for g in gset), [-g for g in gset]))
    cand = [e for e in range(cE.size) if e // n in best]
    bestK = max(itertools.combinations(cand, K),
                key=lambda es: (sum(float(cE[e]) for e in es), [-e for e in sorted(es)]))
    return set(best), set(bestK)


@pytest.mark.parametrize("shape", [(16, 4, 2, 4), (8, 2, 1, 2), (12, 3, 2, 3), (16, 4, 4, 6)])
def test_route_exhaustive(shape):
    E, G, KG, K = shape
    z = synth.normal(40 * E, 1, 21 + E, 1.5).reshape(40, E)
    bias = synth.uniform(E, 1, 22 + E, -0.1, 0.1)
    cfg = O.Cfg(32, E, G, KG, K, 32, 0, 2.5)
    ids, w, fl, s, c = O.route(cfg, z, bias, want_scores=True)
    n = E // G
    for t in range(40):
        gbest, ebest = _brute_route(c[t], G, KG, K)
        assert set(ids[t]) == ebest
        assert {e // n for e in ids[t]} <= gbest
        # slot order: c descending
        assert all(c[t, ids[t, k]] >= c[t, ids[t, k + 1]] for k in range(K - 1))
        # weights: unbiased s, normalised, scaled
        sw = s[t, ids[t]].astype(np.float64)
        assert np.allclose(w[t], sw / sw.sum() * 2.5, rtol=2 * U, atol=0)
        assert np.all(w[t] > 0)
        assert abs(float(w[t].astype(np.float64).sum()) - 2.5) <= 4 * K * U * 2.5


def test_route_special_cases():
    # G == topk_group: plain top-K of biased scores with lower-index ties
    E, K = 16, 5
    z = synth.normal(10 * E, 2, 31, 1.0).reshape(10, E)
    bias = synth.uniform(E, 2, 32, -0.1, 0.1)
    ids, w, fl, s, c = O.route(O.Cfg(32, E, 4, 4, K, 32, 0, 1.0), z, bias, want_scores=True)
    for t in range(10):
        order = np.lexsort((np.arange(E), -c[t].astype(np.float64)))
        assert list(ids[t]) == list(order[:K])
    # K = E with zero bias selects every expert
    ids, w, fl = O.route(O.Cfg(32, 8, 2, 2, 8, 32, 0, 2.5), z[:, :8], np.zeros(8, np.float32))
    assert all(sorted(ids[t]) == list(range(8)) for t in range(10))
    # x = 0: z = 0, s = 1/2, selection by bias then lowest index, w = rsf/K exactly
    zz = np.zeros((3, 256), np.float32)
    b = synth.zipf_pmf(256, 1.1, 0, 5)
    ids, w, fl = O.route(O.Cfg(32, 256, 8, 4, 8, 32, 0, 2.5), zz, b)
    assert np.all(w == np.float32(2.5 / 8)) and np.float32(2.5 / 8) == np.float32(0.3125)
    c0 = (np.float32(0.5) + b).astype(np.float32)
    gs = np.array([np.sort(c0[g * 32:(g + 1) * 32])[-2:].sum(dtype=np.float32) for g in range(8)])
    keep = np.lexsort((np.arange(8), -gs.astype(np.float64)))[:4]
    cand = np.array([e for e in range(256) if e // 32 in keep])
    top = cand[np.lexsort((cand, -c0[cand].astype(np.float64)))][:8]
    assert list(ids[0]) == list(top)


def test_route_near_tie_flags():
    # two candidates 5e-7 apart at the K boundary -> flagged; 1e-4 apart -> not
    z = np.zeros((2, 8), np.float32)
    bias = np.array([0.3, 0.2, 0.1, 0.0, -0.1, -0.2, -0.3, -0.4], np.float32)
    b1 = bias.copy()
    b1[2] = np.float32(0.2) - np.float32(5e-7)
    b2 = bias.copy()
    b2[2] = np.float32(0.2) - np.float32(1e-4)
    cfg = O.Cfg(32, 8, 2, 2, 2, 32, 0, 1.0)
    _, _, f1 = O.route(cfg, z[:1], b1)
    _, _, f2 = O.route(cfg, z[:1], b2)
    assert f1[0] & O.TIE_EXPERT and not (f2[0] & O.TIE_EXPERT)
    b3 = bias.copy()
    b3[1] = np.float32(0.3) - np.float32(5e-7)
    _, _, f3 = O.route(cfg, z[:1], b3)
    assert f3[0] & O.TIE_ORDER


@pytest.mark.parametrize("i", range(3))
def test_topp_golden(i):
    g = HW["topp_cases"]["cases"][i]
    keep, w = O.topp_weights(np.array(g["s_sel"], np.float32), g["topp"], g["rsf"])
    assert np.array_equal(keep, np.array(g["keep"], np.int32))
    assert np.array_equal(w, np.array(g["w"], np.float32))


def test_topp_off_is_the_router_weighting_and_tiny_p_keeps_one():
    sh = synth.TINY
    cfg = O.Cfg.of(sh)
    x = synth.hidden_states(sh, 16, seed=40)
    ids, w, _, sc, _ = O.route(cfg, O.router_logits(x, synth.router_weights(sh)), synth.router_bias(sh),
                               want_scores=True)
    for t in range(16):
        s_sel = sc[t, ids[t]]
        for off in (0.0, 1.0, 1.5, -0.25):
            keep, ww = O.topp_weights(s_sel, off, sh.rsf)
            assert keep.all() and np.array_equal(ww, w[t])
        keep, ww = O.topp_weights(s_sel, 1e-9, sh.rsf)
        assert keep.sum() == 1 and ww[keep == 1][0] == np.float32(sh.rsf)
        assert np.argmax(keep) == np.argmax(s_sel)  # first maximum: the lower slot on ties


@pytest.mark.parametrize("topp", [0.3, 0.7, 0.9])
def test_topp_keeps_the_shortest_heaviest_prefix(topp):
    rng = np.random.default_rng(int(topp * 100))
    for _ in range(200):
        K = int(rng.integers(1, 17))
        s_sel = rng.uniform(0.01, 1.0, K).astype(np.float32)
        if K > 3:
            s_sel[2] = s_sel[1]  # a tie
        keep, w = O.topp_weights(s_sel, topp, 2.5)
        q = s_sel.astype(np.float64) / s_sel.astype(np.float64).sum()
        order = sorted(range(K), key=lambda k: (-q[k], k))
        m = int(keep.sum())
        assert m >= 1 and set(np.nonzero(keep)[0]) == set(order[:m])
        cum = q[order[:m]].sum()
        assert cum >= np.float32(topp) - 1e-12 or m == K
        assert q[order[:m - 1]].sum() < np.float32(topp) + 1e-12
        assert np.all(w[keep == 0] == 0) and np.all(w[keep == 1] > 0)
        assert abs(float(w.astype(np.float64).sum()) - 2.5) <= 2.5 * K * 2.0 ** -23


def test_route_with_topp_drops_slots_of_the_full_selection():
    sh = synth.TINY
    x = synth.hidden_states(sh, 32, seed=41)
    z = O.router_logits(x, synth.router_weights(sh))
    ids0, w0, f0 = O.route(O.Cfg.of(sh), z, synth.router_bias(sh))
    ids, w, f = O.route(O.Cfg.of(sh, topp=0.6), z, synth.router_bias(sh))
    assert np.array_equal(f, f0)
    kept = ids >= 0
    assert np.array_equal(ids[kept], ids0[kept]) and np.all(w[~kept] == 0)
    assert kept.any(1).all() and (~kept).any()  # every token keeps a slot; some slots drop


def test_dispatch_with_dropped_slots_vs_sort():
    rng = np.random.default_rng(8)
    T, K, E = 40, 4, 16
    ids = rng.integers(0, E, (T, K)).astype(np.int32)
    ids[rng.random((T, K)) < 0.3] = -1
    d = O.dispatch(ids, E)
    flat = ids.ravel()
    valid = np.nonzero(flat >= 0)[0]
    order = valid[np.argsort(flat[valid], kind="stable")]
    n = valid.size
    assert d["offsets"][E] == n and np.array_equal(d["sorted_slots"][:n], order)
    assert np.all(d["sorted_slots"][n:] == -1)
    assert np.all(d["slot_pos"][flat < 0] == -1)
    assert np.array_equal(d["slot_pos"][order], np.arange(n))
    assert np.array_equal(d["counts"], np.bincount(flat[valid], minlength=E))
    with pytest.raises(ValueError):
        O.dispatch(np.full((2, 2), -2, np.int32), E)


def test_combine_skips_dropped_slots():
    rng = np.random.default_rng(9)
    T, K, H = 5, 4, 64
    er = rng.normal(size=(T, K, H)).astype(np.float32)
    es = rng.normal(size=(1, T, H)).astype(np.float32)
    w = rng.uniform(0.1, 1.0, (T, K)).astype(np.float32)
    ids = np.zeros((T, K), np.int32)
    assert np.array_equal(O.combine(er, es, w, ids), O.combine(er, es, w))
    ids[:, 1] = -1
    er2 = er.copy()
    er2[:, 1] = np.nan  # a dropped slot's row is never read
    w2 = w.copy()
    w2[:, 1] = 0.0
    ref = O.combine(np.delete(er, 1, axis=1), es, np.delete(w2, 1, axis=1))
    assert np.array_equal(O.combine(er2, es, w2, ids), ref)


def test_route_rejects_bad_shapes():
    with pytest.raises(ValueError):
        O.route(O.Cfg(32, 10, 4, 2, 2, 32, 0, 1.0), np.zeros((1, 10), np.float32), np.zeros(10, np.float32))
    with pytest.raises(ValueError):
        O.route(O.Cfg(32, 8, 4, 1, 3, 32, 0, 1.0), np.zeros((1, 8), np.float32), np.zeros(8, np.float32))


# ----------------------------------------------------------------- dispatch

@pytest.mark.parametrize("T,K,E", [(8, 4, 16), (1, 8, 256), (33, 8, 256), (5, 2, 3)])
def test_dispatch_vs_sort(T, K, E):
    rng = np.random.default_rng(T * 1000 + E)
    ids = rng.integers(0, E, size=(T, K)).astype(np.int32)
    if E > 8:
        ids[0, 0] = ids[0, 1] = 2 if K > 1 else ids[0, 0]
    d = O.dispatch(ids, E)
    flat = ids.reshape(-1)
    ref = [j for (e, j) in sorted((int(flat[j]), j) for j in range(flat.size))]
    assert list(d["sorted_slots"]) == ref
    assert np.array_equal(d["counts"], np.bincount(flat, minlength=E))
    assert d["offsets"][0] == 0 and d["offsets"][-1] == T * K
    assert np.array_equal(np.diff(d["offsets"]), d["counts"])
    assert np.array_equal(d["sorted_slots"][d["slot_pos"]], np.arange(T * K))
    u = np.unique(flat)
    assert d["n_unique"] == u.size and np.array_equal(d["unique_ids"][:u.size], u)


# ------------------------------------------------------------- dots and FFN

def test_block_sums_exact():
    rng = np.random.default_rng(3)
    a = rng.integers(-8, 8, 32 * 200).astype(np.int8)
    b = rng.integers(-127, 128, 32 * 200).astype(np.int8)
    a[:32] = -8
    b[:32] = -127
    S = O.block_sums(a, b)
    ref = (a.astype(np.int64) * b.astype(np.int64)).reshape(-1, 32).sum(1)
    assert np.array_equal(S.astype(np.int64), ref)
    assert S[0] == 32 * 8 * 127


def test_dot_golden_order():
    g = HW["dot_order"]
    q4 = np.zeros(96, np.int8)
    q8 = np.zeros(96, np.int8)
    for b in range(3):
        q4[32 * b] = 1
        q8[32 * b] = g["block_sums"][b]
    v = O.dot_q4q8(q4, g["srow"], q8, np.array(g["d8"], np.float32))
    assert v == np.float32(g["expected"])


@pytest.mark.parametrize("case", ["dot_single_chain", "dot_single_chain_halves", "dot_fused_step"])
def test_dot_golden_single_chain(case):
    g = HW[case]
    nb = g["n_blocks"]
    q4 = np.zeros(32 * nb, np.int8)
    q8 = np.zeros(32 * nb, np.int8)
    for b in range(nb):
        q4[32 * b] = 1
        q8[32 * b] = g["block_sums"][b]
    v = O.dot_q4q8(q4, g["srow"], q8, np.array(g["d8"], np.float32))
    assert v == np.float32(g["expected"])


def test_dot_vs_dequantized_fp64_bound():
    rng = np.random.default_rng(5)
    for n in (64, 2048, 6144):
        for _ in range(20):
            q4 = rng.integers(-7, 8, n).astype(np.int8)
            x = synth.normal(n, int(rng.integers(1 << 30)), 99, 1.0)
            q8, d8 = O.q8_0(x)
            s = np.float32(rng.uniform(0.001, 0.01))
            v = O.dot_q4q8(q4, s, q8, d8)
            terms = d8.astype(np.float64) * (q4.astype(np.int64) * q8.astype(np.int64)).reshape(-1, 32).sum(1)
            exact = float(s) * float(np.sum(terms))
            bound = gamma(n // 32 + 1) * float(s) * float(np.abs(terms).sum())
            assert abs(float(v) - exact) <= bound
            # a dropped block is caught by the same check
            if n >= 64:
                drop = float(s) * float(np.sum(terms[:-1]))
                if abs(drop - exact) > 10 * bound:
                    assert abs(float(v) - drop) > bound


def test_dot_closed_form_constant():
    n = 6144
    q4 = np.ones(n, np.int8)
    for cval in (0.75, -1.5):
        q8, d8 = O.q8_0(np.full(n, cval, np.float32))
        assert np.all(q8 == np.sign(cval) * 127) and np.all(d8 == np.float32(abs(cval) / 127))
        v = O.dot_q4q8(q4, 0.01, q8, d8)
        exact = 0.01 * n * cval
        assert abs(float(v) - exact) <= gamma(n // 32 + 2) * abs(exact) + 1e-9


@pytest.mark.parametrize("case", ["dot_grouped_hand", "dot_grouped_scale_product"])
def test_dot_grouped_golden(case):
    g = HW[case]
    nb = g["n_blocks"]
    q4 = np.zeros(32 * nb, np.int8)
    q8 = np.zeros(32 * nb, np.int8)
    for b in range(nb):
        q4[32 * b] = 1
        q8[32 * b] = g["block_sums"][b]
    v = O.dot_q4q8_grouped(q4, np.array(g["sg"], np.float32), g["group"], q8, np.array(g["d8"], np.float32))
    assert v == np.float32(g["expected"])


@pytest.mark.parametrize("case", ["dot_order", "dot_single_chain", "dot_single_chain_halves"])
def test_dot_grouped_equal_power_of_two_scales_is_per_row_dot(case):
    """Equal group scales that are a power of two scale every product exactly, so the grouped dot equals the
    per-row dot with that row scale bit for bit; on the hand-worked chain goldens this pins the block order."""
    g = HW[case]
    nb = g.get("n_blocks", 3)
    q4 = np.zeros(32 * nb, np.int8)
    q8 = np.zeros(32 * nb, np.int8)
    for b in range(nb):
        q4[32 * b] = 1
        q8[32 * b] = g["block_sums"][b]
    d8 = np.array(g["d8"], np.float32)
    for sigma in (1.0, 0.25, 8.0):
        for group in (32, 32 * nb):
            sg = np.full(nb * 32 // group, sigma, np.float32)
            v = O.dot_q4q8_grouped(q4, sg, group, q8, d8)
            assert v == O.dot_q4q8(q4, sigma, q8, d8)
            if sigma == 1.0 and g.get("srow") == 1.0:
                assert v == np.float32(g["expected"])


def test_dot_grouped_vs_dequantized_fp64_bound():
    rng = np.random.default_rng(15)
    for n, group in ((64, 32), (2048, 32), (2048, 128), (6144, 64)):
        for _ in range(10):
            q4 = rng.integers(-7, 8, n).astype(np.int8)
            x = synth.normal(n, int(rng.integers(1 << 30)), 98, 1.0)
            q8, d8 = O.q8_0(x)
            sg = rng.uniform(0.001, 0.01, n // group).astype(np.float32)
            v = O.dot_q4q8_grouped(q4, sg, group, q8, d8)
            S = (q4.astype(np.int64) * q8.astype(np.int64)).reshape(-1, 32).sum(1)
            sb = np.repeat(sg, group // 32).astype(np.float64)
            terms = d8.astype(np.float64) * sb * S
            exact = float(np.sum(terms))
            bound = gamma(n // 32 + 2) * float(np.abs(terms).sum())
            assert abs(float(v) - exact) <= bound
            # the group of a block matters: scales taken per block index instead would be caught
            if n // group > 1:
                wrong = float(np.sum(d8.astype(np.float64) * np.resize(sg, n // 32).astype(np.float64) * S))
                if abs(wrong - exact) > 10 * bound:
                    assert abs(float(v) - wrong) > bound


def test_swiglu_special_cases():
    assert O.swiglu(0.0, 5.0) == 0.0
    assert O.swiglu(30.0, 1.5) == np.float32(45.0)
    assert O.swiglu(-100.0, 2.0) == np.float32(-200.0 / (1 + math.exp(100.0))) or abs(O.swiglu(-100.0, 2.0)) < 1e-40
    rng = np.random.default_rng(8)
    for _ in range(2000):
        g, u = np.float32(rng.normal(0, 3)), np.float32(rng.normal(0, 3))
        ref = np.float32(float(g) * float(u) * scipy.special.expit(float(g)))
        assert abs(O.swiglu(g, u) - ref) <= np.spacing(abs(ref)) + 1e-45


def test_expert_token_vs_brute_force():
    H, I = 256, 128
    q13, s13 = O.quant_int4_rows(synth.expert_w13(synth.TINY, 3))
    q2, s2 = O.quant_int4_rows(synth.expert_w2(synth.TINY, 3))
    x = synth.hidden_states(synth.TINY, 1)[0]
    qx, dx = O.q8_0(x)
    r = O.expert_token(q13, s13, q2, s2, qx, dx, want_sums=True)
    # exact integer block sums
    S13 = (q13.astype(np.int64) * qx.astype(np.int64)[None]).reshape(2 * I, H // 32, 32).sum(2)
    assert np.array_equal(r["S13"].astype(np.int64), S13)
    # gate/up vs dequantized fp64, within the dot bound
    terms = S13 * dx.astype(np.float64)[None]
    gu = s13.astype(np.float64) * terms.sum(1)
    bound = gamma(H // 32 + 1) * s13.astype(np.float64) * np.abs(terms).sum(1)
    g64, u64 = gu[:I], gu[I:]
    # h = silu(g) u within the propagated bound (a few ulps plus dot error)
    href = g64 * u64 * scipy.special.expit(g64)
    dh_bound = (np.abs(u64) * 1.2 * bound[:I] + np.abs(g64) * bound[I:] + 4 * U * np.abs(href) + 1e-30)
    assert np.all(np.abs(r["h"].astype(np.float64) - href) <= dh_bound)
    qh, dh = O.q8_0(r["h"])
    assert np.array_equal(qh, r["qh"]) and np.array_equal(dh, r["dh"])
    S2 = (q2.astype(np.int64) * r["qh"].astype(np.int64)[None]).reshape(H, I // 32, 32).sum(2)
    assert np.array_equal(r["S2"].astype(np.int64), S2)
    t2 = S2 * r["dh"].astype(np.float64)[None]
    out = s2.astype(np.float64) * t2.sum(1)
    assert np.all(np.abs(r["out"] - out) <= gamma(I // 32 + 1) * s2 * np.abs(t2).sum(1) + 1e-30)


def test_combine_golden_and_bound():
    g = HW["combine_order"]
    y = O.combine(np.array(g["e"], np.float32).reshape(1, 2, 1), np.array([[[g["shared"]]]], np.float32),
                  np.array([g["w"]], np.float32))
    assert y[0, 0] == np.float32(g["expected"])
    rng = np.random.default_rng(9)
    T, K, H = 4, 8, 64
    er = rng.normal(size=(T, K, H)).astype(np.float32)
    es = rng.normal(size=(2, T, H)).astype(np.float32)
    w = rng.uniform(0, 1, size=(T, K)).astype(np.float32)
    y = O.combine(er, es, w)
    ref = es.astype(np.float64).sum(0) + np.einsum("tk,tkh->th", w.astype(np.float64), er.astype(np.float64))
    mag = np.abs(es).sum(0) + np.einsum("tk,tkh->th", w, np.abs(er))
    assert np.all(np.abs(y - ref) <= gamma(K + 2) * mag)
    y0 = O.combine(er, None, w)
    assert np.all(np.abs(y0 - (ref - es.astype(np.float64).sum(0))) <= gamma(K + 1) * mag)
    y1 = O.combine(er[:, :1], es[:1], np.ones((T, 1), np.float32))
    assert np.array_equal(y1, (es[0] + er[:, 0]).astype(np.float32))


# --------------------------------------------------------------- whole layer

def _tiny_layer():
    sh = synth.TINY
    q13, s13, q2, s2 = [], [], [], []
    for e in range(sh.n_experts):
        a, b = O.quant_int4_rows(synth.expert_w13(sh, e))
        q13.append(a)
        s13.append(b)
        a, b = O.quant_int4_rows(synth.expert_w2(sh, e))
        q2.append(a)
        s2.append(b)
    sq13, ss13 = O.quant_int4_rows(synth.shared_w13(sh, 0))
    sq2, ss2 = O.quant_int4_rows(synth.shared_w2(sh, 0))
    return O.LayerQ(synth.router_weights(sh), synth.router_bias(sh), np.stack(q13), np.stack(s13), np.stack(q2),
                    np.stack(s2), sq13[None], ss13[None], sq2[None], ss2[None])


@pytest.fixture(scope="module")
def tiny():
    return _tiny_layer()


def test_layer_teacher_forced_brute_force(tiny):
    sh = synth.TINY
    cfg = O.Cfg.of(sh)
    T, K, H, I = 8, sh.top_k, sh.hidden, sh.inter
    x = synth.hidden_states(sh, T)
    y, t = O.layer_forward(cfg, x, tiny)
    qx, dx = O.q8_0(x)
    assert np.array_equal(t["qx"], qx) and np.array_equal(t["dx"], dx)
    ids, w, fl = O.route(cfg, O.router_logits(x, tiny.router_w), tiny.bias)
    assert np.array_equal(t["ids"], ids) and np.array_equal(t["w"], w)
    # e_out per (token, expert) vs dequantized fp64 given the integer codes
    for tt in range(T):
        for k in range(K + 1):
            row = tt * K + k if k < K else T * K + tt
            if k < K:
                e = ids[tt, k]
                Q2, S2s = tiny.q2[e], tiny.s2[e]
            else:
                Q2, S2s = tiny.sq2[0], tiny.ss2[0]
            S = (Q2.astype(np.int64) * t["qh"][row].astype(np.int64)[None]).reshape(H, I // 32, 32).sum(2)
            terms = S * t["dh"][row].astype(np.float64)[None]
            ref = S2s.astype(np.float64) * terms.sum(1)
            assert np.all(np.abs(t["e_out"][row] - ref) <= gamma(I // 32 + 1) * S2s * np.abs(terms).sum(1) + 1e-30)
    er = t["e_out"][:T * K].reshape(T, K, H).astype(np.float64)
    ref = t["e_out"][T * K:].astype(np.float64) + np.einsum("tk,tkh->th", w.astype(np.float64), er)
    mag = np.abs(t["e_out"][T * K:]) + np.einsum("tk,tkh->th", w, np.abs(er))
    assert np.all(np.abs(y - ref) <= gamma(K + 2) * mag)


def test_layer_batch_invariance_and_permutation(tiny):
    sh = synth.TINY
    cfg = O.Cfg.of(sh)
    x = synth.hidden_states(sh, 8, seed=4)
    y = O.layer_forward(cfg, x, tiny, taps=False)
    for t in range(8):
        assert np.array_equal(O.layer_forward(cfg, x[t:t + 1], tiny, taps=False)[0], y[t])
    perm = np.array([3, 0, 7, 1, 6, 2, 5, 4])
    assert np.array_equal(O.layer_forward(cfg, x[perm], tiny, taps=False), y[perm])


def test_layer_grouped_matches_per_pair_evaluation():
    """The layer with grouped scales equals its pieces evaluated one (token, expert) pair at a time on sliced
    arrays (router, Q8_0, grouped expert FFN, combine): pins the layer's per-expert scale strides."""
    sh = synth.TINY
    G = 64
    cfg = O.Cfg.of(sh, group=G)
    parts = []
    for e in range(sh.n_experts):
        parts.append(O.quant_int4_grouped(synth.expert_w13(sh, e), G) + O.quant_int4_grouped(synth.expert_w2(sh, e), G))
    sh13, shs13 = O.quant_int4_grouped(synth.shared_w13(sh, 0), G)
    sh2, shs2 = O.quant_int4_grouped(synth.shared_w2(sh, 0), G)
    L = O.LayerQ(synth.router_weights(sh), synth.router_bias(sh), np.stack([p[0] for p in parts]),
                 np.stack([p[1] for p in parts]), np.stack([p[2] for p in parts]), np.stack([p[3] for p in parts]),
                 sh13[None], shs13[None], sh2[None], shs2[None])
    x = synth.hidden_states(sh, 6, seed=12)
    y, t = O.layer_forward(cfg, x, L)
    ids, w, _ = O.route(cfg, O.router_logits(x, L.router_w), L.bias)
    for tt in range(6):
        qx, dx = O.q8_0(x[tt])
        rows = [O.expert_token(*parts[e], qx, dx)["out"] for e in ids[tt]]
        shr = O.expert_token(sh13, shs13, sh2, shs2, qx, dx)["out"]
        for k in range(sh.top_k):
            assert np.array_equal(t["e_out"][tt * sh.top_k + k], rows[k])
        yy = O.combine(np.stack(rows)[None], shr[None, None], w[tt:tt + 1])[0]
        assert np.array_equal(y[tt], yy)
    # and differs from the per-row layer of the same weights
    y_row = O.layer_forward(O.Cfg.of(sh), x, _tiny_layer(), taps=False)
    assert not np.array_equal(y, y_row)


def test_layer_topp_matches_per_pair_evaluation(tiny):
    """With adaptive top-p the layer computes only the kept slots and combines them with the renormalised
    weights: equal to per-pair evaluation of the kept (token, expert) pairs and the combine over them."""
    sh = synth.TINY
    cfg = O.Cfg.of(sh, topp=0.55)
    x = synth.hidden_states(sh, 12, seed=13)
    y, t = O.layer_forward(cfg, x, tiny)
    ids, w, _ = O.route(cfg, O.router_logits(x, tiny.router_w), tiny.bias)
    assert np.array_equal(t["ids"], ids) and (ids < 0).any()
    for tt in range(12):
        qx, dx = O.q8_0(x[tt])
        rows = []
        for k in range(sh.top_k):
            e = ids[tt, k]
            r = np.zeros(sh.hidden, np.float32) if e < 0 else \
                O.expert_token(tiny.q13[e], tiny.s13[e], tiny.q2[e], tiny.s2[e], qx, dx)["out"]
            assert np.array_equal(t["e_out"][tt * sh.top_k + k], r)
            rows.append(r)
        shr = O.expert_token(tiny.sq13[0], tiny.ss13[0], tiny.sq2[0], tiny.ss2[0], qx, dx)["out"]
        yy = O.combine(np.stack(rows)[None], shr[None, None], w[tt:tt + 1], ids[tt:tt + 1])
        assert np.array_equal(y[tt], yy[0])


def test_layer_zero_input_closed_form(tiny):
    sh = synth.TINY
    cfg = O.Cfg.of(sh)
    y, t = O.layer_forward(cfg, np.zeros((3, sh.hidden), np.float32), tiny)
    assert not y.any() and not t["h"].any() and not t["qh"].any()
    assert np.all(t["w"] == np.float32(sh.rsf / sh.top_k))


# ----------------------------------------------------------------------- LRU

@pytest.mark.parametrize("name", ["lru_trace", "lru_overflow"])
def test_lru_golden(name):
    g = HW[name]
    L = O.LRU(g["E"], g["slots"])
    for s, need in enumerate(g["steps"]):
        r = L.step(s, need)
        assert list(r["hit"]) == g["expected_hits"][s]
        assert list(r["slot"]) == g["expected_slots"][s]
        assert list(r["evicted"]) == g["expected_evicted"][s]
        if "expected_wait_for" in g:
            assert list(r["wait_for"]) == g["expected_wait_for"][s]
    if "expected_counters" in g:
        assert L.counters() == g["expected_counters"]


def test_lru_single_requests_match_textbook_lru():
    rng = np.random.default_rng(12)
    for cap in (1, 3, 8):
        L = O.LRU(16, cap)
        od = OrderedDict()
        for s in range(400):
            e = int(rng.integers(0, 16))
            r = L.step(s, [e])
            hit = e in od
            if hit:
                od.move_to_end(e)
            else:
                if len(od) >= cap:
                    od.popitem(last=False)
                od[e] = True
            assert bool(r["hit"][0]) == hit


def test_lru_invariants_and_large_capacity():
    rng = np.random.default_rng(13)
    E, S = 64, 16
    L = O.LRU(E, S)
    seen, total = set(), 0
    for s in range(60):
        need = np.unique(rng.zipf(1.3, size=24) % E)
        r = L.step(s, need)
        total += need.size
        res = L.resident()
        assert (res >= 0).sum() <= S
        assert len(set(res[res >= 0].tolist())) == (res >= 0).sum()
        assert np.all(r["slot"] >= 0) and np.all(r["slot"] < S)
    c = L.counters()
    assert c["hits"] + c["misses"] == total
    # capacity >= E: only cold misses
    L = O.LRU(E, E)
    for s in range(30):
        need = np.unique(rng.integers(0, E, size=10))
        L.step(s, need)
        seen |= set(need.tolist())
    assert L.counters()["misses"] == len(seen) and L.counters()["evictions"] == 0


def test_lru_pin_golden():
    g = HW["lru_pin_trace"]
    L = O.LRU(g["E"], g["slots"])
    for s, (need, cnt) in enumerate(zip(g["steps_before_pin"], g["counts_before_pin"])):
        L.step(s, need)
        L.record_usage(need, cnt)
    assert list(L.usage()) == g["expected_usage"]
    p = L.pin_hottest(g["n_pin"])
    assert list(p["pinned"]) == g["expected_pinned"]
    assert list(p["slot"]) == g["expected_pin_slots"]
    assert list(p["loaded"]) == g["expected_pin_loaded"]
    assert list(p["evicted"]) == g["expected_pin_evicted"]
    r = L.step(len(g["steps_before_pin"]), g["step_after_pin"])
    assert list(r["hit"]) == g["expected_hits"]
    assert list(r["slot"]) == g["expected_slots"]
    assert list(r["evicted"]) == g["expected_evicted"]
    assert list(r["wait_for"]) == g["expected_wait_for"]
    assert L.counters() == g["expected_counters"]
    assert list(L.resident()) == g["expected_resident"]


def test_lru_pin_picks_most_used_lower_id_on_ties():
    rng = np.random.default_rng(21)
    E, S = 40, 12
    for trial in range(20):
        L = O.LRU(E, S)
        usage = rng.integers(0, 6, size=E).astype(np.int64)  # small range: many ties
        L.set_usage(usage)
        assert np.array_equal(L.usage(), usage)
        n = int(rng.integers(0, S))
        p = L.pin_hottest(n)
        want = np.lexsort((np.arange(E), -usage))[:n]
        assert np.array_equal(p["pinned"], np.sort(want))
        assert np.all(p["loaded"])  # the cache was empty: every pin is loaded into a free slot
        assert sorted(p["slot"].tolist()) == list(range(n))
    with pytest.raises(ValueError):
        O.LRU(E, S).pin_hottest(S)


def test_lru_pinned_experts_stay_and_hit():
    rng = np.random.default_rng(22)
    E, S, P = 64, 16, 6
    L = O.LRU(E, S)
    for s in range(20):  # learn
        need = np.unique(rng.zipf(1.3, size=24) % E)
        L.step(s, need)
        L.record_usage(need, rng.integers(1, 5, size=need.size))
    p = L.pin_hottest(P)
    pinned = dict(zip(p["pinned"].tolist(), p["slot"].tolist()))
    for s in range(20, 80):
        need = np.unique(rng.zipf(1.3, size=24) % E)
        r = L.step(s, need)
        res = L.resident()
        for e, sl in pinned.items():
            assert res[e] == sl  # never moved or evicted
        for e, h, ev, wf in zip(r["needed"], r["hit"], r["evicted"], r["wait_for"]):
            if int(e) in pinned:
                assert h
            assert int(ev) not in pinned and int(wf) not in pinned
        assert (res >= 0).sum() <= S


def test_lru_pins_leave_a_textbook_lru_on_the_other_slots():
    """Single requests: pinned experts always hit; the rest behave as a textbook LRU of S - P slots."""
    rng = np.random.default_rng(23)
    E, S = 16, 5
    for P in (1, 2, 4):
        L = O.LRU(E, S)
        usage = np.zeros(E, np.int64)
        usage[[3, 7, 11, 13][:P]] = [9, 8, 7, 6][:P]
        L.set_usage(usage)
        pinned = set(L.pin_hottest(P)["pinned"].tolist())
        od = OrderedDict()
        for s in range(400):
            e = int(rng.integers(0, E))
            r = L.step(s, [e])
            if e in pinned:
                assert r["hit"][0]
                continue
            hit = e in od
            if hit:
                od.move_to_end(e)
            else:
                if len(od) >= S - P:
                    od.popitem(last=False)
                od[e] = True
            assert bool(r["hit"][0]) == hit


# ---------------------------------------------------------------- page sizes

def test_page_size_arithmetic():
    g = json.load(open(os.path.join(GOLD, "page_sizes.json")))
    H, I = g["hidden"], g["inter"]
    per_expert = 3 * H * I // 2 + 4 * (2 * I + H)
    assert per_expert == 18_915_328
    assert abs(per_expert / 1e6 - g["mb_per_expert_int4"]) < 0.5
    per_token = g["moe_layers"] * g["experts_per_token_per_layer"] * per_expert
    assert abs(per_token / 1e9 - g["gb_changed_per_token"]) / g["gb_changed_per_token"] < 0.05
    assert abs(g["routed_experts_total"] * per_expert / 1e9 - g["gb_on_disk"]) / g["gb_on_disk"] < 0.05
    assert g["routed_experts_total"] == (g["moe_layers"] + 1) * g["experts_per_layer"]


# ------------------------------------------------------- where several results are correct

def _f32_nearest(fr):
    """The fp32 value nearest to the exact rational fr (ties to even), by exact comparison with its neighbours."""
    from fractions import Fraction
    f = np.float32(float(fr))
    best = None
    for cand in (np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))):
        d = abs(Fraction(float(cand)) - fr)
        key = (d, int(np.float32(cand).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, cand)
    return np.float32(best[1])


def test_router_boundary_flags_constructed():
    # 1 + 2^-24 is the exact midpoint of 1 and 1 + 2^-23: flagged; 1 + 2^-20 is an fp32 value: not flagged
    x = np.array([[1.0, 1.0]], np.float32)
    W = np.array([[1.0, 2.0 ** -24], [1.0, 2.0 ** -20]], np.float32)
    z, fl = O.router_logits_boundary(x, W)
    assert list(fl[0]) == [1, 0]
    assert z[0, 1] == np.float32(1.0 + 2.0 ** -20)
    assert np.array_equal(z, O.router_logits(x, W))


def test_router_boundary_flags_cover_every_rounding_change():
    """Where a logit is not flagged, the correctly rounded exact sum (fractions) is the oracle's logit; flagged
    logits are rare on the GLM-like value range."""
    from fractions import Fraction
    x = synth.normal(6 * 256, 0, 21, 1.0).reshape(6, 256)
    W = synth.normal(40 * 256, 0, 22, 0.02).reshape(40, 256)
    z, fl = O.router_logits_boundary(x, W)
    for t in range(6):
        for e in range(40):
            exact = sum((Fraction(float(a)) * Fraction(float(b)) for a, b in zip(x[t], W[e])), Fraction(0))
            if not fl[t, e]:
                assert z[t, e] == _f32_nearest(exact), (t, e)
    assert fl.mean() < 0.02


def test_swiglu_boundary_constructed():
    # g = 64 + 2^-6, u = 1 + 2^-12: exp(-g) vanishes against 1 in fp64, so the value is g*u = 64 + 2^-5 + 2^-18
    # exactly, the midpoint of two fp32 neighbours (ulp 2^-17 at 64): flagged. u = 1 gives g, an fp32 value.
    g = np.array([64 + 2.0 ** -6, 64 + 2.0 ** -6, 0.0], np.float32)
    u = np.array([1 + 2.0 ** -12, 1.0, 3.0], np.float32)
    assert list(O.swiglu_boundary(g, u)) == [1, 0, 0]


def test_swiglu_boundary_vs_long_double():
    """Unflagged SwiGLU values equal the extended-precision value rounded once to fp32."""
    rng = np.random.default_rng(31)
    g = rng.normal(0, 3, 20000).astype(np.float32)
    u = rng.normal(0, 3, 20000).astype(np.float32)
    fl = O.swiglu_boundary(g, u)
    gl, ul = g.astype(np.longdouble), u.astype(np.longdouble)
    ref = (gl * ul / (np.longdouble(1) + np.exp(-gl))).astype(np.float32)
    got = np.array([O.swiglu(a, b) for a, b in zip(g, u)], np.float32)
    ok = fl == 0
    assert np.array_equal(got[ok].view(np.uint32), ref[ok].view(np.uint32))
    assert fl.sum() <= 2


@pytest.mark.parametrize("group", [0, 64])
def test_gateup_and_down_compose_the_expert(group):
    sh = synth.TINY
    w13, w2 = synth.expert_w13(sh, 2), synth.expert_w2(sh, 2)
    if group:
        q13, s13 = O.quant_int4_grouped(w13, group)
        q2, s2 = O.quant_int4_grouped(w2, group)
    else:
        (q13, s13), (q2, s2) = O.quant_int4_rows(w13), O.quant_int4_rows(w2)
    x = synth.hidden_states(sh, 2, step=3)
    for t in range(2):
        qx, dx = O.q8_0(x[t])
        r = O.expert_token(q13, s13, q2, s2, qx, dx)
        g, u = O.gateup_token(q13, s13, qx, dx)
        h = np.array([O.swiglu(a, b) for a, b in zip(g, u)], np.float32)
        assert np.array_equal(h.view(np.uint32), r["h"].view(np.uint32))
        out = O.down_token(q2, s2, r["qh"], r["dh"])
        assert np.array_equal(out.view(np.uint32), r["out"].view(np.uint32))
        # the gate value of row 0 is the plain dot of its row
        ref = O.dot_q4q8_grouped(q13[0], s13[0], group, qx, dx) if group else O.dot_q4q8(q13[0], s13[0], qx, dx)
        assert g[0] == ref


def test_tie_choice_checker_on_hand_ties():
    """The validity check used for near-tie tokens accepts a choice inside the tie set and refuses others."""
    from tests.harness import tie_choice_ok
    g = HW["router_expert_tie"]  # experts 1, 2 and 4 tie at c = 0.625; the oracle takes 1 and 2
    sh = synth.Shape(32, g["E"], g["G"], g["topk_group"], g["K"], 32, 0, g["rsf"])
    ids, w, fl, s, c = _route_one(g["E"], g["G"], g["topk_group"], g["K"], g["rsf"], g["z"], g["bias"])
    assert tie_choice_ok(sh, c[0], ids[0], [1, 2])[0]
    assert tie_choice_ok(sh, c[0], ids[0], [1, 4])[0]   # another expert of the tie
    assert tie_choice_ok(sh, c[0], ids[0], [2, 1])[0]   # slot order inside the tie
    assert not tie_choice_ok(sh, c[0], ids[0], [1, 3])[0]  # expert 3 scores 0.5: no tie
    assert not tie_choice_ok(sh, c[0], ids[0], [1, 1])[0]
    g = HW["router_group_tie"]  # both groups score 1.125; the oracle keeps group 0 (experts 0, 1)
    sh = synth.Shape(32, g["E"], g["G"], g["topk_group"], g["K"], 32, 0, g["rsf"])
    ids, w, fl, s, c = _route_one(g["E"], g["G"], g["topk_group"], g["K"], g["rsf"], g["z"], g["bias"])
    assert tie_choice_ok(sh, c[0], ids[0], [2, 3])[0]   # the other group of the tie
    assert not tie_choice_ok(sh, c[0], ids[0], [0, 2])[0]  # two groups when one is kept
    g = HW["router_clear"]  # no tie at all: only the oracle's own choice passes
    sh = synth.Shape(32, g["E"], g["G"], g["topk_group"], g["K"], 32, 0, g["rsf"])
    ids, w, fl, s, c = _route_one(g["E"], g["G"], g["topk_group"], g["K"], g["rsf"], g["z"], g["bias"])
    assert tie_choice_ok(sh, c[0], ids[0], list(ids[0]))[0]
    assert not tie_choice_ok(sh, c[0], ids[0], [3, 2])[0]
    assert not tie_choice_ok(sh, c[0], ids[0], [0, 1])[0]
