"""Seeded synthetic inputs shared by the oracle side and the GPU side.

This module holds no arithmetic of the method (no quantisation, routing,
dot products or combines).  It only draws numbers:

* expert weights  N(0, 0.02)   [F][D] gate, [F][D] up, [D][F] down
* activations     N(0, 1)      [T][D]
* router logits   N(0, 1)      [T][E]
* router bias     N(0, 0.1)    [E] per layer
* deep-stack inputs: hidden state N(0, 1) and Zipf(1.1)-skewed logits

The normal draws come from the counter-based generator defined in
synth_host.c (host) and synth_device.hip (device), which agree bit for bit,
so the multi-GB expert tables can be generated on the device while the
oracle regenerates only the experts it needs on the host.

Workload shapes follow the colibri pages: 256 routed experts per MoE layer
plus one shared expert, 8 selected per token ("colibri 소개" and "Bottleneck"
sections of the jeff.news and discuss.pytorch.kr pages); ~19 MB per int4
expert, which d_model=6144, d_ff=2048 reproduce.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, replace

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
HOST_LIB = os.path.join(_HERE, "libsynth_host.so")
DEVICE_LIB = os.path.join(_HERE, "libsynth_device.so")

# Stream-id fields: kind (8 bits) | family (8) | layer (16) | tag (32)
KIND_WEIGHT = 1
KIND_X = 2
KIND_LOGIT = 3
KIND_BIAS = 4
KIND_HIDDEN = 5
KIND_PERM = 6
KIND_GUMBEL = 7
KIND_ROUTER = 8

SEED = 0
W_SIGMA = 0.02
X_SIGMA = 1.0
LOGIT_SIGMA = 1.0
BIAS_SIGMA = 0.1
ZIPF_S = 1.1


def stream_id(kind: int, family: int, layer: int = 0, tag: int = 0) -> int:
    assert 0 <= kind < 256 and 0 <= family < 256 and 0 <= layer < 65536 and 0 <= tag < 2**32
    return (kind << 56) | (family << 48) | (layer << 32) | tag


@dataclass(frozen=True)
class Workload:
    """One synthetic workload: layer shape, routing and token count."""
    name: str
    D: int          # d_model
    F: int          # d_ff per expert
    E: int          # routed experts
    S: int          # shared experts (0 or 1)
    k: int          # experts selected per token
    T: int          # tokens per pass
    family: int     # weight family (layers of one family share streams)
    tag: int        # separates the token/logit draws of different workloads
    layers: int = 1
    steps: int = 1  # sequential passes (deep decode stack)
    zipf: bool = False
    bias: bool = True

    @property
    def bytes_per_expert(self) -> int:
        # gate + up: [F][D/2] u8 + [F] f32 each; down: [D][F/2] u8 + [D] f32
        return 2 * (self.F * self.D // 2 + 4 * self.F) + (self.D * self.F // 2 + 4 * self.D)


WORKLOADS = {
    0: Workload("tiny-layer d256 f128 e16+1 top2 t4", 256, 128, 16, 1, 2, 4, family=0, tag=0),
    1: Workload("decode d6144 f2048 e256+1 top8 t1", 6144, 2048, 256, 1, 8, 1, family=1, tag=1),
    2: Workload("verify d6144 f2048 e256+1 top8 t4", 6144, 2048, 256, 1, 8, 4, family=1, tag=2),
    3: Workload("prefill d6144 f2048 e256+1 top8 t2048", 6144, 2048, 256, 1, 8, 2048, family=1, tag=3),
    4: Workload("deep-decode 40 layers d6144 f2048 e256+1 top8 zipf1.1 256 tokens", 6144, 2048,
                256, 1, 8, 1, family=1, tag=4, layers=40, steps=256, zipf=True),
}


def bias_free(w: Workload) -> Workload:
    """The prefill workload with zero router bias (the 'uniform-ish' reading)."""
    return replace(w, name=w.name + " bias-free", bias=False, tag=w.tag + 100)


# ----------------------------------------------------------------------------
# host generator
_host = None


def _host_lib():
    global _host
    if _host is None:
        if not os.path.exists(HOST_LIB):
            raise RuntimeError(f"{HOST_LIB} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(HOST_LIB)
        lib.synth_normal.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64,
                                     ctypes.c_int64, ctypes.c_float, ctypes.c_void_p]
        lib.synth_normal.restype = None
        lib.synth_uniform.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64,
                                      ctypes.c_int64, ctypes.c_void_p]
        lib.synth_uniform.restype = None
        _host = lib
    return _host


def normal(sid: int, n: int, sigma: float, offset: int = 0, seed: int = SEED) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    if n:
        _host_lib().synth_normal(seed, sid, offset, n, sigma, out.ctypes.data)
    return out


def uniform(sid: int, n: int, offset: int = 0, seed: int = SEED) -> np.ndarray:
    out = np.empty(n, dtype=np.float64)
    if n:
        _host_lib().synth_uniform(seed, sid, offset, n, out.ctypes.data)
    return out


# ----------------------------------------------------------------------------
# device generator
_dev = None


def _dev_lib():
    global _dev
    if _dev is None:
        if not os.path.exists(DEVICE_LIB):
            raise RuntimeError(f"{DEVICE_LIB} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(DEVICE_LIB)
        lib.synth_normal_device.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64,
                                            ctypes.c_int64, ctypes.c_float, ctypes.c_void_p,
                                            ctypes.c_void_p]
        lib.synth_normal_device.restype = ctypes.c_int
        _dev = lib
    return _dev


def normal_device(sid: int, n: int, sigma: float, out_ptr: int, stream_ptr: int,
                  offset: int = 0, seed: int = SEED) -> None:
    rc = _dev_lib().synth_normal_device(seed, sid, offset, n, sigma, out_ptr, stream_ptr)
    if rc != 0:
        raise RuntimeError(f"synth_normal_device failed with hipError {rc}")


# ----------------------------------------------------------------------------
# workload recipes
MATRIX_GATE, MATRIX_UP, MATRIX_DOWN = 0, 1, 2


def weight_shape(w: Workload, matrix: int):
    return (w.F, w.D) if matrix in (MATRIX_GATE, MATRIX_UP) else (w.D, w.F)


def weight_stream(w: Workload, layer: int, expert: int, matrix: int) -> int:
    return stream_id(KIND_WEIGHT, w.family, layer, expert * 4 + matrix)


def weight_host(w: Workload, layer: int, expert: int, matrix: int) -> np.ndarray:
    """fp32 weights of one matrix of one expert (expert index E is the shared one)."""
    rows, cols = weight_shape(w, matrix)
    return normal(weight_stream(w, layer, expert, matrix), rows * cols, W_SIGMA).reshape(rows, cols)


def weight_device(w: Workload, layer: int, expert: int, matrix: int, out_ptr: int,
                  stream_ptr: int) -> None:
    rows, cols = weight_shape(w, matrix)
    normal_device(weight_stream(w, layer, expert, matrix), rows * cols, W_SIGMA, out_ptr, stream_ptr)


def activations(w: Workload, T: int, token0: int = 0, layer: int = 0) -> np.ndarray:
    return normal(stream_id(KIND_X, w.family, layer, w.tag), T * w.D, X_SIGMA,
                  offset=token0 * w.D).reshape(T, w.D)


def router_bias(w: Workload, layer: int = 0) -> np.ndarray:
    if not w.bias:
        return np.zeros(w.E, dtype=np.float32)
    return normal(stream_id(KIND_BIAS, w.family, layer, 0), w.E, BIAS_SIGMA)


def logits(w: Workload, T: int, token0: int = 0, layer: int = 0) -> np.ndarray:
    """Router logits for T tokens: N(0, 1), or Zipf(1.1)-skewed for the deep stack."""
    if w.zipf:
        return zipf_logits(w, layer, T, token0)
    return normal(stream_id(KIND_LOGIT, w.family, layer, w.tag), T * w.E, LOGIT_SIGMA,
                  offset=token0 * w.E).reshape(T, w.E)


def expert_ranks(w: Workload, layer: int) -> np.ndarray:
    """A seeded permutation: rank (1..E) of every expert in this layer's popularity order."""
    u = uniform(stream_id(KIND_PERM, w.family, layer, w.tag), w.E)
    order = np.argsort(u, kind="stable")
    ranks = np.empty(w.E, dtype=np.int64)
    ranks[order] = np.arange(1, w.E + 1)
    return ranks


def zipf_logits(w: Workload, layer: int, T: int, token0: int = 0) -> np.ndarray:
    """log-weight of a Zipf(s) law over a seeded expert ranking plus Gumbel(0,1) noise.

    Taking the top-k of log-weights plus independent Gumbel noise samples k
    experts without replacement with probability proportional to rank^-s, so
    hot experts recur from token to token as in the pages' cache-hit reports.
    """
    ranks = expert_ranks(w, layer)
    u = uniform(stream_id(KIND_GUMBEL, w.family, layer, w.tag), T * w.E,
                offset=token0 * w.E).reshape(T, w.E)
    g = -np.log(-np.log(u))
    return (-ZIPF_S * np.log(ranks.astype(np.float64))[None, :] + g).astype(np.float32)


def router_weights(w: Workload, layer: int = 0) -> np.ndarray:
    """F32 router projection [E][D] of one layer: N(0, 0.02)."""
    return normal(stream_id(KIND_ROUTER, w.family, layer, 0), w.E * w.D, W_SIGMA).reshape(w.E, w.D)


def hidden0(w: Workload, T: int, token0: int = 0) -> np.ndarray:
    """Initial fp32 hidden state of the deep decode stack."""
    return normal(stream_id(KIND_HIDDEN, w.family, 0, w.tag), T * w.D, X_SIGMA,
                  offset=token0 * w.D).reshape(T, w.D)
