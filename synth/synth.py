"""Seeded synthetic inputs for the MoE-layer tests and bench.

This module generates random inputs only: fp32 normals and uniforms from a
counter-based stream (synth.h), the Zipf popularity used as the router
correction bias, and the correlated hidden states of an MTP-verify batch. It
holds none of the MoE method's arithmetic, and both the oracle side and the
GPU side draw their inputs from it.

Host fills come from libsynth_host.so (gcc); device fills from
libsynth_gpu.so (hipcc). Both evaluate the same per-element definition and
agree bit for bit (checked by the tests).

Workload shapes (the colibrì pages: GLM-5.2 routes each token to 8 of 256
experts per layer, about 19 MB of int4 per expert; the tiny shape is a
seconds-scale check of the same structure):
  tiny:  H=256,  E=16,  G=4, topk_group=2, K=4, I=128,  1 shared, rsf 2.5
  glm:   H=6144, E=256, G=8, topk_group=4, K=8, I=2048, 1 shared, rsf 2.5
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))

ROUTER_W, BIAS_U, BIAS_PERM, W13, W2, SH_W13, SH_W2, X, X_SHARED, X_POS = range(1, 11)


def stream_id(kind: int, layer: int = 0, index: int = 0) -> int:
    return (kind << 24) | ((layer & 0xFFF) << 12) | (index & 0xFFF)


@dataclass(frozen=True)
class Shape:
    hidden: int
    n_experts: int
    n_group: int
    topk_group: int
    top_k: int
    inter: int
    n_shared: int
    rsf: float
    w_sigma: float = 0.02
    bias_kind: str = "zipf"  # "uniform" (U(-0.1, 0.1)) or "zipf" (s = 1.1)


TINY = Shape(256, 16, 4, 2, 4, 128, 1, 2.5, bias_kind="uniform")
GLM = Shape(6144, 256, 8, 4, 8, 2048, 1, 2.5, bias_kind="zipf")

_host = None
_gpu = None


def host_lib():
    global _host
    if _host is None:
        lib = ctypes.CDLL(os.path.join(_HERE, "libsynth_host.so"))
        lib.synth_philox.argtypes = [ctypes.c_void_p] * 3
        lib.synth_normal_f32.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64, ctypes.c_uint32,
                                         ctypes.c_uint32, ctypes.c_double]
        lib.synth_uniform_f32.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64, ctypes.c_uint32,
                                          ctypes.c_uint32, ctypes.c_double, ctypes.c_double]
        lib.synth_permutation.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint32, ctypes.c_uint32]
        lib.synth_zipf_pmf.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_double, ctypes.c_uint32,
                                       ctypes.c_uint32]
        _host = lib
    return _host


def gpu_lib():
    global _gpu
    if _gpu is None:
        lib = ctypes.CDLL(os.path.join(_HERE, "libsynth_gpu.so"))
        lib.synth_gpu_normal_f32.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64, ctypes.c_uint32,
                                             ctypes.c_uint32, ctypes.c_double, ctypes.c_void_p]
        lib.synth_gpu_uniform_f32.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64, ctypes.c_uint32,
                                              ctypes.c_uint32, ctypes.c_double, ctypes.c_double, ctypes.c_void_p]
        _gpu = lib
    return _gpu


def philox(ctr, key):
    c = (ctypes.c_uint32 * 4)(*ctr)
    k = (ctypes.c_uint32 * 2)(*key)
    o = (ctypes.c_uint32 * 4)()
    host_lib().synth_philox(c, k, o)
    return [int(v) for v in o]


def normal(n: int, seed: int, stream: int, sigma: float = 1.0, start: int = 0) -> np.ndarray:
    out = np.empty(int(n), np.float32)
    host_lib().synth_normal_f32(out.ctypes.data, int(n), int(start), seed, stream, float(sigma))
    return out


def uniform(n: int, seed: int, stream: int, lo: float, hi: float, start: int = 0) -> np.ndarray:
    out = np.empty(int(n), np.float32)
    host_lib().synth_uniform_f32(out.ctypes.data, int(n), int(start), seed, stream, float(lo), float(hi))
    return out


def permutation(n: int, seed: int, stream: int) -> np.ndarray:
    out = np.empty(int(n), np.int32)
    host_lib().synth_permutation(out.ctypes.data, int(n), seed, stream)
    return out


def zipf_pmf(n: int, s: float, seed: int, stream: int) -> np.ndarray:
    out = np.empty(int(n), np.float32)
    host_lib().synth_zipf_pmf(out.ctypes.data, int(n), float(s), seed, stream)
    return out


# ---------------------------------------------------------------- layer inputs

def router_weights(shape: Shape, seed: int = 0, layer: int = 0) -> np.ndarray:
    """[E][H] fp32 from N(0, 0.02)."""
    E, H = shape.n_experts, shape.hidden
    return normal(E * H, seed, stream_id(ROUTER_W, layer), shape.w_sigma).reshape(E, H)


def router_bias(shape: Shape, seed: int = 0, layer: int = 0) -> np.ndarray:
    """Correction bias [E]: U(-0.1, 0.1), or the Zipf(s=1.1) popularity over a seeded permutation of experts."""
    E = shape.n_experts
    if shape.bias_kind == "uniform":
        return uniform(E, seed, stream_id(BIAS_U, layer), -0.1, 0.1)
    return zipf_pmf(E, 1.1, seed, stream_id(BIAS_PERM, layer))


def expert_w13(shape: Shape, e: int, seed: int = 0, layer: int = 0) -> np.ndarray:
    """Routed expert e: [2I][H] fp32 (gate rows 0..I-1, up rows I..2I-1) from N(0, 0.02)."""
    return normal(2 * shape.inter * shape.hidden, seed, stream_id(W13, layer, e), shape.w_sigma).reshape(
        2 * shape.inter, shape.hidden)


def expert_w2(shape: Shape, e: int, seed: int = 0, layer: int = 0) -> np.ndarray:
    """Routed expert e: down projection [H][I] fp32 from N(0, 0.02)."""
    return normal(shape.hidden * shape.inter, seed, stream_id(W2, layer, e), shape.w_sigma).reshape(
        shape.hidden, shape.inter)


def shared_w13(shape: Shape, s: int, seed: int = 0, layer: int = 0) -> np.ndarray:
    return normal(2 * shape.inter * shape.hidden, seed, stream_id(SH_W13, layer, s), shape.w_sigma).reshape(
        2 * shape.inter, shape.hidden)


def shared_w2(shape: Shape, s: int, seed: int = 0, layer: int = 0) -> np.ndarray:
    return normal(shape.hidden * shape.inter, seed, stream_id(SH_W2, layer, s), shape.w_sigma).reshape(
        shape.hidden, shape.inter)


def hidden_states(shape: Shape, T: int, seed: int = 0, layer: int = 0, step: int = 0) -> np.ndarray:
    """[T][H] fp32 from N(0, 1)."""
    return normal(T * shape.hidden, seed, stream_id(X, layer, step), 1.0).reshape(T, shape.hidden)


def mtp_hidden_states(shape: Shape, n_seq: int, n_pos: int, rho: float = 0.8, seed: int = 0, layer: int = 0,
                      step: int = 0) -> np.ndarray:
    """MTP-verify batch: n_seq sequences x n_pos positions, token t = n_pos*s + p.

    x[s,p,:] = sqrt(rho) * c[s,:] + sqrt(1-rho) * z[s,p,:] with c, z ~ N(0,1), so positions of one
    sequence have pairwise correlation rho (equicorrelated); evaluated in fp64, rounded to fp32.
    """
    H = shape.hidden
    c = normal(n_seq * H, seed, stream_id(X_SHARED, layer, step), 1.0).reshape(n_seq, 1, H).astype(np.float64)
    z = normal(n_seq * n_pos * H, seed, stream_id(X_POS, layer, step), 1.0).reshape(n_seq, n_pos, H).astype(
        np.float64)
    x = math.sqrt(rho) * c + math.sqrt(1.0 - rho) * z
    return x.reshape(n_seq * n_pos, H).astype(np.float32)


# ----------------------------------------------------------------- device fills

def gpu_normal_(t, seed: int, stream: int, sigma: float = 1.0, start: int = 0, cuda_stream: int = 0):
    """Fill a contiguous float32 CUDA tensor in place with the same values normal() gives."""
    assert t.is_contiguous() and str(t.dtype) == "torch.float32" and t.is_cuda
    rc = gpu_lib().synth_gpu_normal_f32(ctypes.c_void_p(t.data_ptr()), t.numel(), int(start), seed, stream,
                                        float(sigma), ctypes.c_void_p(cuda_stream))
    if rc != 0:
        raise RuntimeError(f"synth_gpu_normal_f32 failed: hip error {rc}")
    return t
