"""Seeded synthetic inputs for the routed-expert FP8 MoE prefill layer.

Shared by the CPU oracle's tests and the GPU path's tests and bench.  It holds
no arithmetic of the method: it writes an FP8 layer (codes + FP32 128x128 block
scales), BF16 hidden rows and top-k routing decisions, all as pure functions
of (seed, tensor, index), see ``gen.c``.

Workload shapes follow the layers the pages discuss: a GLM-class routed-expert
layer (E=256, top-8, H=6144, I=2048; "ktransformers #2244", Design: one 9.002
GiB slot holds all 256 experts' gate/up/down FP8 codes and scales) and one
GPU's tensor-sliced share of a GLM-4.6 layer (I=192 per rank, zero-padded to
256; "hpc-ops #80", gap table row 6).
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libmoegen.so")
_lib = None

ROUTE_SOFTMAX = 0
ROUTE_SIGMOID_NORMAL = 1
ROUTE_SIGMOID_UNIFORM = 2
ROUTE_ZIPF = 3


def build(force: bool = True) -> str:
    """Compile gen.c into libmoegen.so (gcc, OpenMP)."""
    src = os.path.join(_HERE, "gen.c")
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(src):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               src, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        lib.gen_layer.argtypes = [ctypes.c_uint64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                  ctypes.c_int32, ctypes.c_int32, ctypes.c_float, P, P, P, P, P, P]
        lib.gen_layer.restype = None
        lib.gen_tokens.argtypes = [ctypes.c_uint64, ctypes.c_int64, ctypes.c_int32, ctypes.c_double,
                                   ctypes.c_float, P, P]
        lib.gen_tokens.restype = None
        lib.gen_routing.argtypes = [ctypes.c_uint64, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                    ctypes.c_int32, ctypes.c_int32, ctypes.c_double, P, P]
        lib.gen_routing.restype = None
        lib.gen_logits.argtypes = [ctypes.c_uint64, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                   ctypes.c_int32, ctypes.c_double, P]
        lib.gen_logits.restype = None
        _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return ctypes.c_void_p(a.ctypes.data)


@dataclasses.dataclass
class Layer:
    """Canonical FP8 layer, as handed to the method.

    gate, up: u8[E][I][H]; down: u8[E][H][I] (rows = output features);
    gate_scale, up_scale: f32[E][ceil(I/128)][H/128];
    down_scale: f32[E][H/128][ceil(I/128)].
    """
    E: int
    H: int
    I: int
    gate: np.ndarray
    up: np.ndarray
    down: np.ndarray
    gate_scale: np.ndarray
    up_scale: np.ndarray
    down_scale: np.ndarray

    @property
    def nbytes(self) -> int:
        return sum(a.nbytes for a in (self.gate, self.up, self.down,
                                      self.gate_scale, self.up_scale, self.down_scale))


def make_layer(E: int, H: int, I: int, seed: int = 0, stddev: float = 0.02,
               e_begin: int = 0, e_end: int | None = None) -> Layer:
    """Experts [e_begin, e_end) of the seeded layer (weights 0.02*N(0,1),
    quantised per 128x128 block with scale = amax/448)."""
    if e_end is None:
        e_end = E
    n = e_end - e_begin
    nI, nH = (I + 127) // 128, (H + 127) // 128
    gate = np.empty((n, I, H), np.uint8)
    up = np.empty((n, I, H), np.uint8)
    down = np.empty((n, H, I), np.uint8)
    gs = np.empty((n, nI, nH), np.float32)
    us = np.empty((n, nI, nH), np.float32)
    ds = np.empty((n, nH, nI), np.float32)
    _load().gen_layer(seed, E, H, I, e_begin, e_end, stddev, _ptr(gate), _ptr(up), _ptr(down),
                      _ptr(gs), _ptr(us), _ptr(ds))
    return Layer(E if (e_begin == 0 and e_end == E) else n, H, I, gate, up, down, gs, us, ds)


def make_tokens(T: int, H: int, seed: int = 0, outlier_frac: float = 0.0,
                outlier_mult: float = 100.0):
    """BF16 rows as uint16[T][H] (N(0,1)); ceil(outlier_frac*T) rows x outlier_mult.
    Returns (x_bits, is_outlier)."""
    x = np.empty((T, H), np.uint16)
    flag = np.empty((max(T, 1),), np.uint8)
    _load().gen_tokens(seed, T, H, outlier_frac, outlier_mult, _ptr(x), _ptr(flag))
    return x, flag[:T].astype(bool)


def make_routing(T: int, E: int, k: int, kind: int, seed: int = 0, n_masked: int = 0,
                 zipf_s: float = 1.2):
    """(ids int32[T][k], w float32[T][k]): top-k ids, descending score, ties to the
    lower id; weights normalised over the chosen slots."""
    if not (1 <= k <= min(E, 64)):
        raise ValueError("need 1 <= k <= min(E, 64)")
    if kind == ROUTE_ZIPF and k > E - n_masked:
        raise ValueError("k larger than the number of unmasked experts")
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    _load().gen_routing(seed, T, E, k, kind, n_masked, zipf_s, _ptr(ids), _ptr(w))
    return ids, w


def make_logits(T: int, E: int, kind: int, seed: int = 0, n_masked: int = 0,
                zipf_s: float = 1.2) -> np.ndarray:
    """Router logits float32[T][E], the same draws ``make_routing`` selects
    from (N(0,1), U(0,1), or Zipf log-popularity + Gumbel with -inf for the
    masked experts), rounded to FP32."""
    logits = np.empty((T, E), np.float32)
    _load().gen_logits(seed, T, E, kind, n_masked, zipf_s, _ptr(logits))
    return logits


def bf16_bits_to_f32(x: np.ndarray) -> np.ndarray:
    """Widen BF16 bit patterns to float32 (exact)."""
    return (x.astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic configuration: layer shape, rows, routing recipe."""
    name: str
    E: int
    k: int
    H: int
    I: int
    T: int
    route: int
    rho: float
    outlier_frac: float
    n_masked: int = 0
    seed: int = 0
    shared: int = 0      # 1: the layer holds E + 1 experts, the last always on


# The five configurations: a tiny layer, the GLM-class layer at 256 / 4096 /
# 8192 rows, and one GPU's 192-wide slice of a GLM-4.6 expert.
TINY = Workload("tiny_e8_k2_h256_i128_t64", 8, 2, 256, 128, 64, ROUTE_SOFTMAX, 1.0, 0.0)
GLM_T256 = Workload("glm_e256_k8_h6144_i2048_t256", 256, 8, 6144, 2048, 256,
                    ROUTE_SIGMOID_NORMAL, 2.5, 0.01)
GLM_T4096 = Workload("glm_e256_k8_h6144_i2048_t4096_uniform", 256, 8, 6144, 2048, 4096,
                     ROUTE_SIGMOID_UNIFORM, 2.5, 0.01)
GLM_T8192_ZIPF = Workload("glm_e256_k8_h6144_i2048_t8192_zipf", 256, 8, 6144, 2048, 8192,
                          ROUTE_ZIPF, 2.5, 0.01, n_masked=8)
SLICE_T16 = Workload("slice_e160_k8_h5120_i192_t16", 160, 8, 5120, 192, 16,
                     ROUTE_SIGMOID_NORMAL, 1.0, 0.01)
SLICE_T64 = dataclasses.replace(SLICE_T16, name="slice_e160_k8_h5120_i192_t64", T=64)
SLICE_T1024 = dataclasses.replace(SLICE_T16, name="slice_e160_k8_h5120_i192_t1024", T=1024)

# Compute-bound probe (not one of the pages' configurations): every token
# routes to all 8 experts of a GLM-shaped layer, so each expert gets T rows
# and the grouped GEMMs run at ~6,100 FLOP per weight byte.
PROBE_T4096 = Workload("probe_e8_k8_h6144_i2048_t4096", 8, 8, 6144, 2048, 4096,
                       ROUTE_SIGMOID_UNIFORM, 1.0, 0.0)

# The GLM-class layer with one always-on shared expert in the same grouped
# GEMMs (nine slots per token over E + 1 experts), at T=256.
GLM_T256_SHARED = dataclasses.replace(GLM_T256, name="glm_e256s1_k8_h6144_i2048_t256", shared=1)

WORKLOADS = {w.name: w for w in (TINY, GLM_T256, GLM_T4096, GLM_T8192_ZIPF,
                                 SLICE_T16, SLICE_T64, SLICE_T1024, PROBE_T4096, GLM_T256_SHARED)}


def make_inputs(wl: Workload):
    """(x_bits uint16[T][H], ids int32[T][k], w float32[T][k], is_outlier bool[T])."""
    x, out = make_tokens(wl.T, wl.H, wl.seed, wl.outlier_frac)
    ids, w = make_routing(wl.T, wl.E, wl.k, wl.route, wl.seed, wl.n_masked)
    return x, ids, w, out
