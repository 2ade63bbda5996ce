"""ctypes binding of libmoe.so (include/moe.h), same names as the C entry points.

Argument marshalling only: tensors are passed as raw device pointers, the HIP
stream as its handle; every step runs in the library's HIP kernels. There is
no fallback: if libmoe.so is missing the import fails.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_OK, MOE_E_NULL, MOE_E_SHAPE, MOE_E_WORKSPACE, MOE_E_HIP, MOE_E_NOMEM, MOE_E_UNSUPPORTED, MOE_E_ARG = (
    0, -1, -2, -3, -4, -5, -6, -7)
MOE_TIE_EXPERT, MOE_TIE_GROUP, MOE_TIE_ORDER = 1, 2, 4
MOE_N_STAGES = 9
STAGES = ("router", "topk", "dispatch", "q8_x", "gateup_gemv", "down_gemv", "gateup_mfma", "down_mfma",
          "combine")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
# torch ships its own HIP runtime under the same soname as the system one; the
# library must bind to the runtime torch uses (tensors and streams come from
# torch), so torch is loaded first whenever it is installed.
try:
    import torch  # noqa: F401
except ImportError:
    pass
_lib = ctypes.CDLL(LIB_PATH)

P, I32, I64, SZ, F32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float


class moe_config(ctypes.Structure):
    _fields_ = [("hidden", I32), ("n_experts", I32), ("n_group", I32), ("topk_group", I32), ("top_k", I32),
                ("inter", I32), ("n_shared", I32), ("routed_scaling_factor", F32), ("gemm_min_tokens", I32),
                ("weight_bits", I32), ("group_size", I32), ("topp", F32)]


class moe_layer_weights(ctypes.Structure):
    _fields_ = [(n, P) for n in ("router_w", "router_bias", "w13", "s13", "w2", "s2", "sh_w13", "sh_s13", "sh_w2",
                                 "sh_s2")]


class moe_taps(ctypes.Structure):
    _fields_ = [("topk_ids", P), ("topk_w", P), ("near_tie", P), ("qx", P), ("dx", P), ("h", P), ("qh", P),
                ("dh", P), ("e_out", P), ("sum_slot", I32), ("gateup_sums", P), ("down_sums", P), ("counts", P),
                ("offsets", P), ("sorted_slots", P), ("slot_pos", P), ("unique_ids", P), ("n_unique", P)]


class moe_host_experts(ctypes.Structure):
    _fields_ = [("w13", P), ("s13", P), ("w2", P), ("s2", P)]


class moe_cache_stats(ctypes.Structure):
    _fields_ = [("hits", I64), ("misses", I64), ("evictions", I64), ("bytes_h2d", I64), ("steps", I64),
                ("h2d_ms", ctypes.c_double), ("pinned", I64)]


def _sig(name, res, args):
    f = getattr(_lib, name)
    f.restype = res
    f.argtypes = args
    return f


_sig("moe_version", I32, [])
_sig("moe_strerror", ctypes.c_char_p, [I32])
_sig("moe_last_hip_error", I32, [])
_sig("moe_workspace_bytes", SZ, [P, I32])
_sig("moe_quantize_int4", I32, [P, I32, I32, P, P, P])
_sig("moe_quantize_int8", I32, [P, I32, I32, P, P, P])
_sig("moe_quantize_int4_grouped", I32, [P, I32, I32, I32, P, P, P])
_sig("moe_quantize_q8_0", I32, [P, I64, P, P, P])
_sig("moe_router", I32, [P, P, I32, P, P, P, P, P, P, SZ, P])
_sig("moe_dispatch", I32, [P, P, I32, P, P, P, P, P, P, P, SZ, P])
_sig("moe_layer_forward", I32, [P, P, P, I32, P, P, SZ, P, P])
_sig("moe_expert_cache_create", I32, [P, I32, I32, ctypes.POINTER(P)])
_sig("moe_expert_cache_forward", I32, [P, P, P, P, I32, P, P, SZ, P, P, P, P])
_sig("moe_expert_cache_stats", I32, [P, P])
_sig("moe_expert_cache_usage", I32, [P, P])
_sig("moe_expert_cache_set_usage", I32, [P, P])
_sig("moe_expert_cache_pin_hottest", I32, [P, I32, P, P])
_sig("moe_expert_cache_destroy", None, [P])
_sig("moe_prof_enable", I32, [I32, ctypes.c_uint32])
_sig("moe_prof_read", I32, [P, I32, P])
_sig("moe_prof_disable", None, [])
_sig("moe_membench_read", I32, [P, SZ, I32, I32, P, P])
_sig("moe_membench_copy", I32, [P, P, SZ, I32, P])

EXPORTED = ("moe_version", "moe_strerror", "moe_last_hip_error", "moe_workspace_bytes", "moe_quantize_int4",
            "moe_quantize_int8", "moe_quantize_int4_grouped", "moe_quantize_q8_0", "moe_router", "moe_dispatch", "moe_layer_forward",
            "moe_expert_cache_create",
            "moe_expert_cache_forward", "moe_expert_cache_stats", "moe_expert_cache_usage", "moe_expert_cache_set_usage",
            "moe_expert_cache_pin_hottest", "moe_expert_cache_destroy", "moe_prof_enable",
            "moe_prof_read", "moe_prof_disable", "moe_membench_read", "moe_membench_copy")


class MoeError(RuntimeError):
    def __init__(self, fn, rc):
        msg = _lib.moe_strerror(rc).decode()
        if rc == MOE_E_HIP:
            msg += f" (hipError {_lib.moe_last_hip_error()})"
        super().__init__(f"{fn}: {msg} [{rc}]")
        self.rc = rc


def _check(fn, rc):
    if rc != MOE_OK:
        raise MoeError(fn, rc)
    return rc


def _ptr(t):
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        import torch
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


@dataclass
class Config:
    hidden: int
    n_experts: int
    n_group: int
    topk_group: int
    top_k: int
    inter: int
    n_shared: int
    routed_scaling_factor: float
    gemm_min_tokens: int = 0
    weight_bits: int = 4
    group_size: int = 0
    topp: float = 0.0

    def c(self):
        return moe_config(self.hidden, self.n_experts, self.n_group, self.topk_group, self.top_k, self.inter,
                          self.n_shared, self.routed_scaling_factor, self.gemm_min_tokens, self.weight_bits,
                          self.group_size, self.topp)


def moe_version():
    return _lib.moe_version()


def moe_workspace_bytes(cfg: Config, max_tokens: int) -> int:
    c = cfg.c()
    return int(_lib.moe_workspace_bytes(ctypes.byref(c), int(max_tokens)))


def moe_quantize_int4(w, packed, scales, stream=None):
    rows, cols = w.shape
    return _check("moe_quantize_int4",
                  _lib.moe_quantize_int4(_ptr(w), rows, cols, _ptr(packed), _ptr(scales), _stream(stream)))


def moe_quantize_int8(w, codes, scales, stream=None):
    rows, cols = w.shape
    return _check("moe_quantize_int8",
                  _lib.moe_quantize_int8(_ptr(w), rows, cols, _ptr(codes), _ptr(scales), _stream(stream)))


def moe_quantize_int4_grouped(w, group, packed, scales, stream=None):
    rows, cols = w.shape
    return _check("moe_quantize_int4_grouped",
                  _lib.moe_quantize_int4_grouped(_ptr(w), rows, cols, int(group), _ptr(packed), _ptr(scales),
                                                 _stream(stream)))


def moe_quantize_q8_0(x, q, d, stream=None):
    return _check("moe_quantize_q8_0", _lib.moe_quantize_q8_0(_ptr(x), x.numel(), _ptr(q), _ptr(d), _stream(stream)))


def moe_router(cfg: Config, x, router_w, router_bias, topk_ids, topk_w, near_tie, ws, stream=None):
    c = cfg.c()
    return _check("moe_router", _lib.moe_router(ctypes.byref(c), _ptr(x), x.shape[0], _ptr(router_w),
                                                _ptr(router_bias), _ptr(topk_ids), _ptr(topk_w), _ptr(near_tie),
                                                _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def moe_dispatch(cfg: Config, topk_ids, counts, offsets, sorted_slots, slot_pos, unique_ids, n_unique, ws,
                 stream=None):
    c = cfg.c()
    return _check("moe_dispatch", _lib.moe_dispatch(ctypes.byref(c), _ptr(topk_ids), topk_ids.shape[0], _ptr(counts),
                                                    _ptr(offsets), _ptr(sorted_slots), _ptr(slot_pos),
                                                    _ptr(unique_ids), _ptr(n_unique), _ptr(ws),
                                                    ws.numel() * ws.element_size(), _stream(stream)))


def layer_weights(router_w, router_bias, w13, s13, w2, s2, sh_w13=None, sh_s13=None, sh_w2=None, sh_s2=None):
    return moe_layer_weights(*[_ptr(t) for t in (router_w, router_bias, w13, s13, w2, s2, sh_w13, sh_s13, sh_w2,
                                                 sh_s2)])


def taps(sum_slot=-1, **bufs):
    t = moe_taps()
    t.sum_slot = sum_slot
    for k, v in bufs.items():
        setattr(t, k, None if v is None else v.data_ptr())
    return t


def moe_layer_forward(cfg: Config, weights: moe_layer_weights, x, y, ws, tap: moe_taps | None = None, stream=None,
                      T: int | None = None):
    c = cfg.c()
    T = x.shape[0] if T is None else T
    return _check("moe_layer_forward",
                  _lib.moe_layer_forward(ctypes.byref(c), ctypes.byref(weights), _ptr(x), T, _ptr(y), _ptr(ws),
                                         ws.numel() * ws.element_size(), ctypes.byref(tap) if tap else None,
                                         _stream(stream)))


def moe_prof_enable(max_calls: int, stages=None):
    """Time the named stages (names from STAGES; None = all) of the next max_calls forwards."""
    mask = 0 if stages is None else sum(1 << STAGES.index(n) for n in stages)
    return _check("moe_prof_enable", _lib.moe_prof_enable(int(max_calls), mask))


def moe_prof_read(max_calls: int):
    import numpy as np
    out = np.zeros((max_calls, MOE_N_STAGES), np.float32)
    n = ctypes.c_int32(0)
    _check("moe_prof_read", _lib.moe_prof_read(out.ctypes.data, max_calls, ctypes.byref(n)))
    return out[:n.value]


def moe_prof_disable():
    _lib.moe_prof_disable()


def moe_membench_read(buf, blocks: int, unroll: int, sink, stream=None):
    return _check("moe_membench_read", _lib.moe_membench_read(_ptr(buf), buf.numel() * buf.element_size(), blocks,
                                                              unroll, _ptr(sink), _stream(stream)))


def moe_membench_copy(src, dst, blocks: int, stream=None):
    return _check("moe_membench_copy", _lib.moe_membench_copy(_ptr(src), _ptr(dst), src.numel() * src.element_size(),
                                                              blocks, _stream(stream)))


class HostExperts:
    """Pointer arrays of moe_host_experts: per expert, pinned host pointers (int) or pinned host tensors (kept
    alive here) for w13, s13, w2, s2."""

    def __init__(self, w13, s13, w2, s2):
        self._keep = (list(w13), list(s13), list(w2), list(s2))
        E = len(self._keep[0])
        arr = ctypes.c_void_p * E
        self._arrs = [arr(*[t if isinstance(t, int) else t.data_ptr() for t in lst]) for lst in self._keep]
        self.c = moe_host_experts(*[ctypes.cast(a, P) for a in self._arrs])


class ExpertCache:
    """moe_expert_cache_* of one layer; destroy() (or garbage collection) releases the slot pool."""

    def __init__(self, cfg: Config, n_slots: int, max_tokens: int):
        self._h = P()
        c = cfg.c()
        _check("moe_expert_cache_create", _lib.moe_expert_cache_create(ctypes.byref(c), int(n_slots),
                                                                        int(max_tokens), ctypes.byref(self._h)))
        self.E = cfg.n_experts

    def forward(self, resident, host: HostExperts, x, y, ws, compute, copy, T=None, trace=False):
        import numpy as np
        T = x.shape[0] if T is None else T
        hit = np.zeros(self.E, np.int8) if trace else None
        slot = np.zeros(self.E, np.int32) if trace else None
        _check("moe_expert_cache_forward",
               _lib.moe_expert_cache_forward(self._h, ctypes.byref(resident), ctypes.byref(host.c), _ptr(x), T,
                                             _ptr(y), _ptr(ws), ws.numel() * ws.element_size(), _stream(compute),
                                             _stream(copy), hit.ctypes.data if trace else None,
                                             slot.ctypes.data if trace else None))
        return (hit, slot) if trace else None

    def stats(self):
        s = moe_cache_stats()
        _check("moe_expert_cache_stats", _lib.moe_expert_cache_stats(self._h, ctypes.byref(s)))
        return dict(hits=s.hits, misses=s.misses, evictions=s.evictions, bytes_h2d=s.bytes_h2d, steps=s.steps,
                    h2d_ms=s.h2d_ms, pinned=s.pinned)

    def usage(self):
        """Positions routed to each expert over every forward (host int64 [E])."""
        import numpy as np
        out = np.zeros(self.E, np.int64)
        _check("moe_expert_cache_usage", _lib.moe_expert_cache_usage(self._h, out.ctypes.data))
        return out

    def set_usage(self, usage):
        import numpy as np
        u = np.ascontiguousarray(usage, dtype=np.int64)
        assert u.shape == (self.E,)
        _check("moe_expert_cache_set_usage", _lib.moe_expert_cache_set_usage(self._h, u.ctypes.data))

    def pin_hottest(self, n_pin: int, host: HostExperts, copy):
        _check("moe_expert_cache_pin_hottest",
               _lib.moe_expert_cache_pin_hottest(self._h, int(n_pin), ctypes.byref(host.c), _stream(copy)))

    def destroy(self):
        if self._h:
            _lib.moe_expert_cache_destroy(self._h)
            self._h = P()

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass
