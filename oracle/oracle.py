"""ctypes + numpy marshalling for the C oracle (liboracle.so).

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the bench's
CPU-baseline leg; never by the product package. Every computation happens in
moe_oracle.c; this file only allocates arrays and passes pointers.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_lib = None

TIE_EXPERT, TIE_GROUP, TIE_ORDER = 1, 2, 4


class OrcCfg(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("n_experts", ctypes.c_int32), ("n_group", ctypes.c_int32),
                ("topk_group", ctypes.c_int32), ("top_k", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("n_shared", ctypes.c_int32), ("rsf", ctypes.c_float), ("group", ctypes.c_int32),
                ("topp", ctypes.c_float)]


class OrcTaps(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("z", "ids", "w", "flags", "qx", "dx", "h", "qh", "dh", "e_out")]


def lib():
    global _lib
    if _lib is None:
        L = ctypes.CDLL(os.path.join(_HERE, "liboracle.so"))
        P, I64, I32, F = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float
        L.orc_quant_int4_rows.argtypes = [P, I64, I64, P, P]
        L.orc_pack_int4.argtypes = [P, I64, P]
        L.orc_unpack_int4.argtypes = [P, I64, P]
        L.orc_unpack_int4_tiled64.argtypes = [P, I64, I64, P]
        L.orc_quant_int8_rows.argtypes = [P, I64, I64, P, P]
        L.orc_unpack_int8_tiled64.argtypes = [P, I64, I64, P]
        L.orc_quant_int4_grouped.argtypes = [P, I64, I64, I64, P, P]
        L.orc_unpack_scales_tiled64.argtypes = [P, I64, I64, P]
        L.orc_dot_q4q8_grouped.argtypes = [P, P, I64, P, P, I64]
        L.orc_dot_q4q8_grouped.restype = F
        L.orc_expert_token_g.argtypes = [I32, I32, I32] + [P] * 12
        L.orc_q8_0.argtypes = [P, I64, P, P]
        L.orc_router_logits.argtypes = [P, I32, I32, P, I32, P]
        L.orc_router_logits_boundary.argtypes = [P, I32, I32, P, I32, P, P]
        L.orc_swiglu_boundary.argtypes = [P, P, I64, P]
        L.orc_gateup_token.argtypes = [I32, I32, I32, P, P, P, P, P, P]
        L.orc_down_token.argtypes = [I32, I32, I32, P, P, P, P, P]
        L.orc_route.argtypes = [P, P, P, I32, P, P, P, P, P]
        L.orc_dispatch.argtypes = [I32, I32, I32, P, P, P, P, P, P, P]
        L.orc_block_sums.argtypes = [P, P, I64, P]
        L.orc_dot_q4q8.argtypes = [P, F, P, P, I64]
        L.orc_dot_q4q8.restype = F
        L.orc_swiglu.argtypes = [F, F]
        L.orc_swiglu.restype = F
        L.orc_expert_token.argtypes = [I32, I32] + [P] * 12
        L.orc_combine.argtypes = [I32, I32, I32, I32, P, P, P, P]
        L.orc_combine_ids.argtypes = [I32, I32, I32, I32, P, P, P, P, P]
        L.orc_topp_weights.argtypes = [P, I32, F, F, P, P]
        L.orc_layer_forward.argtypes = [P, I32] + [P] * 12 + [P]
        L.orc_lru_new.argtypes = [I32, I32]
        L.orc_lru_new.restype = P
        L.orc_lru_free.argtypes = [P]
        L.orc_lru_step.argtypes = [P, I64, P, I32, P, P, P, P]
        L.orc_lru_counters.argtypes = [P, P, P, P]
        L.orc_lru_record_usage.argtypes = [P, P, P, I32]
        L.orc_lru_set_usage.argtypes = [P, P]
        L.orc_lru_usage.argtypes = [P, P]
        L.orc_lru_pin_hottest.argtypes = [P, I32, P, P, P, P]
        L.orc_lru_resident.argtypes = [P, P]
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


@dataclass
class Cfg:
    hidden: int
    n_experts: int
    n_group: int
    topk_group: int
    top_k: int
    inter: int
    n_shared: int
    rsf: float
    group: int = 0  # 0: one weight scale per row; else one per group of this many elements along K
    topp: float = 0.0  # adaptive expert top-p in (0, 1); otherwise off

    def c(self):
        return OrcCfg(self.hidden, self.n_experts, self.n_group, self.topk_group, self.top_k, self.inter,
                      self.n_shared, self.rsf, self.group, self.topp)

    @staticmethod
    def of(shape, group: int = 0, topp: float = 0.0):
        return Cfg(shape.hidden, shape.n_experts, shape.n_group, shape.topk_group, shape.top_k, shape.inter,
                   shape.n_shared, shape.rsf, group, topp)


def quant_int4_rows(w):
    w = _c(w, np.float32)
    rows, cols = w.shape
    q = np.empty((rows, cols), np.int8)
    s = np.empty(rows, np.float32)
    lib().orc_quant_int4_rows(_p(w), rows, cols, _p(q), _p(s))
    return q, s


def pack_int4(q):
    q = _c(q, np.int8).reshape(-1)
    out = np.empty(q.size // 2, np.uint8)
    lib().orc_pack_int4(_p(q), q.size, _p(out))
    return out


def quant_int8_rows(w):
    w = _c(w, np.float32)
    rows, cols = w.shape
    q = np.empty((rows, cols), np.int8)
    sc = np.empty(rows, np.float32)
    lib().orc_quant_int8_rows(_p(w), rows, cols, _p(q), _p(sc))
    return q, sc


def quant_int4_grouped(w, group):
    """(codes [rows][cols] int8, scales [rows][cols/group] fp32)."""
    w = _c(w, np.float32)
    rows, cols = w.shape
    assert group > 0 and cols % group == 0
    q = np.empty((rows, cols), np.int8)
    sc = np.empty((rows, cols // group), np.float32)
    lib().orc_quant_int4_grouped(_p(w), rows, cols, group, _p(q), _p(sc))
    return q, sc


def unpack_scales_tiled64(b, rows, ng):
    b = _c(b, np.float32).reshape(-1)
    assert b.size == rows * ng
    sc = np.empty((rows, ng), np.float32)
    lib().orc_unpack_scales_tiled64(_p(b), rows, ng, _p(sc))
    return sc


def unpack_int8_tiled64(b, rows, cols):
    b = _c(b, np.uint8).reshape(-1)
    assert b.size == rows * cols
    q = np.empty((rows, cols), np.int8)
    lib().orc_unpack_int8_tiled64(_p(b), rows, cols, _p(q))
    return q


def unpack_int4(b, n):
    b = _c(b, np.uint8).reshape(-1)
    q = np.empty(n, np.int8)
    lib().orc_unpack_int4(_p(b), n, _p(q))
    return q


def unpack_int4_tiled64(b, rows, cols):
    b = _c(b, np.uint8).reshape(-1)
    q = np.empty((rows, cols), np.int8)
    lib().orc_unpack_int4_tiled64(_p(b), rows, cols, _p(q))
    return q


def q8_0(v):
    v = _c(v, np.float32)
    shp = v.shape
    n = v.size
    q = np.empty(n, np.int8)
    d = np.empty(n // 32, np.float32)
    lib().orc_q8_0(_p(v), n, _p(q), _p(d))
    return q.reshape(shp), d.reshape(shp[:-1] + (shp[-1] // 32,))


def router_logits(x, Wr):
    x = _c(x, np.float32)
    Wr = _c(Wr, np.float32)
    T, H = x.shape
    E = Wr.shape[0]
    z = np.empty((T, E), np.float32)
    lib().orc_router_logits(_p(x), T, H, _p(Wr), E, _p(z))
    return z


def router_logits_boundary(x, Wr):
    """(z [T][E] as router_logits, flag [T][E] uint8: 1 where another fp64 summation order may round the logit
    to the neighbouring fp32 value)."""
    x = _c(x, np.float32)
    Wr = _c(Wr, np.float32)
    T, H = x.shape
    E = Wr.shape[0]
    z = np.empty((T, E), np.float32)
    fl = np.empty((T, E), np.uint8)
    lib().orc_router_logits_boundary(_p(x), T, H, _p(Wr), E, _p(z), _p(fl))
    return z, fl


def swiglu_boundary(g, u):
    """uint8 flags: 1 where the fp64 SwiGLU of (g, u) lies within 2^-48 (relative) of an fp32 midpoint."""
    g = _c(g, np.float32)
    u = _c(u, np.float32)
    fl = np.empty(g.shape, np.uint8)
    lib().orc_swiglu_boundary(_p(g), _p(u), g.size, _p(fl))
    return fl


def _group_of(H, I, s13, s2):
    if s13.ndim == 2:
        group = H // s13.shape[1]
        assert s13.shape == (2 * I, H // group) and s2.shape == (H, I // group)
        return group
    return 0


def gateup_token(q13, s13, qx, dx):
    """(g [I], u [I]): the gate and up projections of one token (s13 [2I] row scales or [2I][H/G] group scales)."""
    q13 = _c(q13, np.int8)
    s13 = _c(s13, np.float32)
    I2, H = q13.shape
    I = I2 // 2
    group = H // s13.shape[1] if s13.ndim == 2 else 0
    g = np.empty(I, np.float32)
    u = np.empty(I, np.float32)
    lib().orc_gateup_token(H, I, group, _p(q13), _p(s13), _p(_c(qx, np.int8)), _p(_c(dx, np.float32)), _p(g),
                           _p(u))
    return g, u


def down_token(q2, s2, qh, dh):
    """out [H]: the down projection of one token's Q8_0 h (s2 [H] row scales or [H][I/G] group scales)."""
    q2 = _c(q2, np.int8)
    s2 = _c(s2, np.float32)
    H, I = q2.shape
    group = I // s2.shape[1] if s2.ndim == 2 else 0
    out = np.empty(H, np.float32)
    lib().orc_down_token(H, I, group, _p(q2), _p(s2), _p(_c(qh, np.int8)), _p(_c(dh, np.float32)), _p(out))
    return out


def route(cfg: Cfg, z, bias, want_scores=False):
    z = _c(z, np.float32)
    bias = _c(bias, np.float32)
    T = z.shape[0]
    K, E = cfg.top_k, cfg.n_experts
    ids = np.empty((T, K), np.int32)
    w = np.empty((T, K), np.float32)
    fl = np.empty(T, np.uint8)
    s = np.empty((T, E), np.float32) if want_scores else None
    c = np.empty((T, E), np.float32) if want_scores else None
    oc = cfg.c()
    rc = lib().orc_route(ctypes.byref(oc), _p(z), _p(bias), T, _p(ids), _p(w), _p(fl), _p(s), _p(c))
    if rc != 0:
        raise ValueError(f"orc_route: invalid shape (rc={rc})")
    if want_scores:
        return ids, w, fl, s, c
    return ids, w, fl


def topp_weights(s_sel, topp, rsf):
    """(keep [K] int32, w [K] fp32) of K selected slots' unbiased scores under adaptive top-p."""
    s_sel = _c(s_sel, np.float32)
    keep = np.empty(s_sel.size, np.int32)
    w = np.empty(s_sel.size, np.float32)
    lib().orc_topp_weights(_p(s_sel), s_sel.size, float(topp), float(rsf), _p(keep), _p(w))
    return keep, w


def dispatch(ids, E):
    ids = _c(ids, np.int32)
    T, K = ids.shape
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    ss = np.full(T * K, -1, np.int32)  # entries past offsets[E] (slots dropped by top-p) stay -1
    sp = np.empty(T * K, np.int32)
    uq = np.empty(E, np.int32)
    nu = np.zeros(1, np.int32)
    rc = lib().orc_dispatch(T, K, E, _p(ids), _p(counts), _p(offsets), _p(ss), _p(sp), _p(uq), _p(nu))
    if rc != 0:
        raise ValueError("orc_dispatch: expert id out of range")
    return dict(counts=counts, offsets=offsets, sorted_slots=ss, slot_pos=sp, unique_ids=uq,
                n_unique=int(nu[0]))


def block_sums(a, b):
    a = _c(a, np.int8).reshape(-1)
    b = _c(b, np.int8).reshape(-1)
    S = np.empty(a.size // 32, np.int32)
    lib().orc_block_sums(_p(a), _p(b), a.size, _p(S))
    return S


def dot_q4q8(q4, srow, q8, d8):
    q4 = _c(q4, np.int8)
    q8 = _c(q8, np.int8)
    d8 = _c(d8, np.float32)
    return np.float32(lib().orc_dot_q4q8(_p(q4), float(srow), _p(q8), _p(d8), q4.size))


def dot_q4q8_grouped(q4, sg, group, q8, d8):
    q4 = _c(q4, np.int8)
    sg = _c(sg, np.float32)
    q8 = _c(q8, np.int8)
    d8 = _c(d8, np.float32)
    return np.float32(lib().orc_dot_q4q8_grouped(_p(q4), _p(sg), group, _p(q8), _p(d8), q4.size))


def swiglu(g, u):
    return np.float32(lib().orc_swiglu(float(g), float(u)))


def expert_token(q13, s13, q2, s2, qx, dx, want_sums=False):
    """s13 [2I] and s2 [H]: per-row scales; s13 [2I][H/G] and s2 [H][I/G]: grouped scales."""
    q13 = _c(q13, np.int8)
    s13 = _c(s13, np.float32)
    q2 = _c(q2, np.int8)
    s2 = _c(s2, np.float32)
    qx = _c(qx, np.int8)
    dx = _c(dx, np.float32)
    H = q2.shape[0]
    I = q2.shape[1]
    h = np.empty(I, np.float32)
    qh = np.empty(I, np.int8)
    dh = np.empty(I // 32, np.float32)
    out = np.empty(H, np.float32)
    S13 = np.empty((2 * I, H // 32), np.int32) if want_sums else None
    S2 = np.empty((H, I // 32), np.int32) if want_sums else None
    group = _group_of(H, I, s13, s2)
    lib().orc_expert_token_g(H, I, group, _p(q13), _p(s13), _p(q2), _p(s2), _p(qx), _p(dx), _p(h), _p(qh), _p(dh),
                             _p(out), _p(S13), _p(S2))
    r = dict(h=h, qh=qh, dh=dh, out=out)
    if want_sums:
        r.update(S13=S13, S2=S2)
    return r


def combine(e_routed, e_shared, w, ids=None):
    """ids (optional, [T][K]): slots with id -1 add nothing."""
    e_routed = _c(e_routed, np.float32)
    w = _c(w, np.float32)
    T, K, H = e_routed.shape
    NS = 0 if e_shared is None else e_shared.shape[0]
    es = None if e_shared is None else _c(e_shared, np.float32)
    ids = None if ids is None else _c(ids, np.int32)
    y = np.empty((T, H), np.float32)
    lib().orc_combine_ids(T, K, H, NS, _p(e_routed), _p(es), _p(w), _p(ids), _p(y))
    return y


@dataclass
class LayerQ:
    """A layer's weights in the oracle's unpacked form: int8 codes + fp32 scales (per row, or per group with
    Cfg.group > 0: s13 [E][2I][H/G], s2 [E][H][I/G])."""
    router_w: np.ndarray  # [E][H] fp32
    bias: np.ndarray      # [E] fp32
    q13: np.ndarray       # [E][2I][H] int8
    s13: np.ndarray       # [E][2I]
    q2: np.ndarray        # [E][H][I] int8
    s2: np.ndarray        # [E][H]
    sq13: np.ndarray      # [NS][2I][H]
    ss13: np.ndarray
    sq2: np.ndarray
    ss2: np.ndarray


def layer_forward(cfg: Cfg, x, L: LayerQ, taps=True):
    x = _c(x, np.float32)
    T, H = x.shape
    E, K, I, NS = cfg.n_experts, cfg.top_k, cfg.inter, cfg.n_shared
    R = T * K + NS * T
    y = np.empty((T, H), np.float32)
    t = dict(z=np.empty((T, E), np.float32), ids=np.empty((T, K), np.int32), w=np.empty((T, K), np.float32),
             flags=np.empty(T, np.uint8), qx=np.empty((T, H), np.int8), dx=np.empty((T, H // 32), np.float32),
             h=np.empty((R, I), np.float32), qh=np.empty((R, I), np.int8), dh=np.empty((R, I // 32), np.float32),
             e_out=np.empty((R, H), np.float32))
    ot = OrcTaps(*[_p(t[n]) for n in ("z", "ids", "w", "flags", "qx", "dx", "h", "qh", "dh", "e_out")])
    oc = cfg.c()
    arrs = [_c(a, dt) for a, dt in ((L.router_w, np.float32), (L.bias, np.float32), (L.q13, np.int8),
                                     (L.s13, np.float32), (L.q2, np.int8), (L.s2, np.float32),
                                     (L.sq13, np.int8), (L.ss13, np.float32), (L.sq2, np.int8),
                                     (L.ss2, np.float32))]
    rc = lib().orc_layer_forward(ctypes.byref(oc), T, _p(x), *[_p(a) for a in arrs], _p(y), ctypes.byref(ot))
    if rc != 0:
        raise ValueError(f"orc_layer_forward failed rc={rc}")
    return (y, t) if taps else y


class LRU:
    """The oracle's per-layer LRU policy simulator."""

    def __init__(self, n_experts, n_slots):
        self.E = n_experts
        self.h = lib().orc_lru_new(n_experts, n_slots)
        if not self.h:
            raise ValueError("bad LRU shape")

    def step(self, step, needed):
        nd = _c(np.sort(np.asarray(needed)), np.int32)
        n = nd.size
        hit = np.zeros(n, np.uint8)
        slot = np.zeros(n, np.int32)
        ev = np.zeros(n, np.int32)
        wf = np.zeros(n, np.int32)
        rc = lib().orc_lru_step(self.h, step, _p(nd), n, _p(hit), _p(slot), _p(ev), _p(wf))
        if rc != 0:
            raise ValueError("needed list must be unique expert ids")
        return dict(needed=nd, hit=hit.astype(bool), slot=slot, evicted=ev, wait_for=wf)

    def record_usage(self, needed, counts):
        nd = _c(np.asarray(needed), np.int32)
        ct = _c(np.asarray(counts), np.int32)
        lib().orc_lru_record_usage(self.h, _p(nd), _p(ct), nd.size)

    def set_usage(self, usage):
        u = _c(np.asarray(usage), np.int64)
        assert u.size == self.E
        lib().orc_lru_set_usage(self.h, _p(u))

    def usage(self):
        out = np.empty(self.E, np.int64)
        lib().orc_lru_usage(self.h, _p(out))
        return out

    def pin_hottest(self, n_pin):
        ch = np.zeros(max(n_pin, 1), np.int32)
        sl = np.zeros(max(n_pin, 1), np.int32)
        ld = np.zeros(max(n_pin, 1), np.uint8)
        ev = np.zeros(max(n_pin, 1), np.int32)
        rc = lib().orc_lru_pin_hottest(self.h, n_pin, _p(ch), _p(sl), _p(ld), _p(ev))
        if rc != 0:
            raise ValueError("n_pin must be in [0, n_slots)")
        return dict(pinned=ch[:n_pin], slot=sl[:n_pin], loaded=ld[:n_pin].astype(bool), evicted=ev[:n_pin])

    def counters(self):
        a, b, c = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
        lib().orc_lru_counters(self.h, ctypes.byref(a), ctypes.byref(b), ctypes.byref(c))
        return dict(hits=a.value, misses=b.value, evictions=c.value)

    def resident(self):
        out = np.empty(self.E, np.int32)
        lib().orc_lru_resident(self.h, _p(out))
        return out

    def __del__(self):
        if getattr(self, "h", None):
            lib().orc_lru_free(self.h)
            self.h = None
