"""CPU oracle for the routed-expert FP8 MoE prefill layer (ctypes binding).

TEST INFRASTRUCTURE ONLY: imported by tests/, by ``__graft_entry__.smoke()``
and by the CPU-baseline leg of ``bench.py``; never by the product package.
The C source (``oracle.c``) states what each step computes and which passage
of the pages it follows; the pins that tie it to something other than itself
are in ``tests/test_oracle_*.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

FAULTS = {
    "none": 0,
    "weight_scale_index": 1,
    "drop_last_kblock": 2,
    "unstable_plan": 3,
    "silu_clamp": 4,
    "pad_garbage": 5,
    "nan_code_is_nan": 6,
    "group_64": 7,
    "down_scale_transposed": 8,
    "encode_truncate": 9,
    "drop_rho": 10,
    "silu_sign": 11,
    "gate_up_swap": 12,
    "route_tie_high": 13,
    "route_all_experts": 14,
    "shared_inside_rho": 15,
    "slice_scale_block": 16,
    "a16_h_truncate": 17,
}

ROUTE_SOFTMAX = 0
ROUTE_SIGMOID = 1

OUT_BF16 = 0
OUT_F32 = 1


def build(force: bool = True) -> str:
    """Compile oracle.c: gcc -O2, OpenMP, no fast-math, no FP contraction."""
    src = os.path.join(_HERE, "oracle.c")
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(src):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fno-fast-math", "-ffp-contract=off",
                               "-fPIC", "-shared", "-std=c11", src, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class _Layer(ctypes.Structure):
    _fields_ = [("E", ctypes.c_int32), ("H", ctypes.c_int32), ("I", ctypes.c_int32),
                ("gate", ctypes.c_void_p), ("up", ctypes.c_void_p), ("down", ctypes.c_void_p),
                ("gate_scale", ctypes.c_void_p), ("up_scale", ctypes.c_void_p),
                ("down_scale", ctypes.c_void_p)]


class _Debug(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("xq", "sx", "gu", "hq", "sh", "y", "counts", "offsets", "perm", "inv", "hb")]


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        lib.orc_e4m3_decode.argtypes = [ctypes.c_uint32]
        lib.orc_e4m3_decode.restype = ctypes.c_float
        lib.orc_e4m3_encode.argtypes = [ctypes.c_float]
        lib.orc_e4m3_encode.restype = ctypes.c_uint32
        for name in ("orc_decode_array", "orc_encode_array", "orc_bf16_to_f32_array",
                     "orc_f32_to_bf16_array"):
            getattr(lib, name).argtypes = [P, ctypes.c_int64, P]
            getattr(lib, name).restype = None
        lib.orc_quantize_rows.argtypes = [P, ctypes.c_int64, ctypes.c_int64, P, P]
        lib.orc_quantize_rows.restype = None
        lib.orc_plan.argtypes = [P, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, P, P, P, P]
        lib.orc_plan.restype = ctypes.c_int64
        lib.orc_forward.argtypes = [ctypes.POINTER(_Layer), ctypes.c_int32, P, P, P, ctypes.c_int64,
                                    ctypes.c_float, ctypes.c_int32, P, ctypes.POINTER(_Debug),
                                    ctypes.c_int32]
        lib.orc_forward.restype = ctypes.c_int64
        lib.orc_forward_a16.argtypes = lib.orc_forward.argtypes
        lib.orc_forward_a16.restype = ctypes.c_int64
        lib.orc_down_combine.argtypes = [ctypes.POINTER(_Layer), ctypes.c_int32, P, P, P, P,
                                         ctypes.c_int64, ctypes.c_float, ctypes.c_int32, P, P,
                                         ctypes.c_int32]
        lib.orc_down_combine.restype = ctypes.c_int64
        lib.orc_bruteforce_fp64.argtypes = [ctypes.POINTER(_Layer), ctypes.c_int32, P, P, P,
                                            ctypes.c_int64, ctypes.c_double, ctypes.c_int32, P,
                                            ctypes.c_int32]
        lib.orc_bruteforce_fp64.restype = ctypes.c_int32
        lib.orc_set_fault.argtypes = [ctypes.c_int32]
        lib.orc_set_fault.restype = None
        lib.orc_max_threads.argtypes = []
        lib.orc_max_threads.restype = ctypes.c_int32
        lib.orc_slice_matrix.argtypes = [P, P, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32,
                                         ctypes.c_int64, ctypes.c_int64, P, P]
        lib.orc_slice_matrix.restype = ctypes.c_int32
        lib.orc_set_activation_limit.argtypes = [ctypes.c_float]
        lib.orc_set_activation_limit.restype = None
        lib.orc_route.argtypes = [P, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, P, P]
        lib.orc_route.restype = ctypes.c_int32
        lib.orc_silu_mul_array.argtypes = [P, P, ctypes.c_int64, P]
        lib.orc_silu_mul_array.restype = None
        _lib = lib
    return _lib


def _p(a):
    if a is None:
        return None
    assert isinstance(a, np.ndarray) and a.flags["C_CONTIGUOUS"], "need a C-contiguous array"
    return ctypes.c_void_p(a.ctypes.data)


def set_activation_limit(limit: float) -> None:
    """Clamped SiLU limit L for forward / bruteforce_fp64 (0 = unclamped)."""
    _load().orc_set_activation_limit(float(limit))


def set_fault(name: str) -> None:
    """Plant a deliberate mistake in the oracle (for testing the pins only)."""
    _load().orc_set_fault(FAULTS[name])


def max_threads() -> int:
    return int(_load().orc_max_threads())


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(c.shape, np.float32)
    _load().orc_decode_array(_p(c), c.size, _p(out))
    return out


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    f = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(f.shape, np.uint8)
    _load().orc_encode_array(_p(f), f.size, _p(out))
    return out


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    u = np.ascontiguousarray(b, dtype=np.uint16)
    out = np.empty(u.shape, np.float32)
    _load().orc_bf16_to_f32_array(_p(u), u.size, _p(out))
    return out


def f32_to_bf16(f: np.ndarray) -> np.ndarray:
    v = np.ascontiguousarray(f, dtype=np.float32)
    out = np.empty(v.shape, np.uint16)
    _load().orc_f32_to_bf16_array(_p(v), v.size, _p(out))
    return out


def silu_mul(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    """h = silu(g) * u elementwise in FP32, as the layer computes it (with
    the activation limit currently set)."""
    g = np.ascontiguousarray(g, dtype=np.float32)
    u = np.ascontiguousarray(u, dtype=np.float32)
    out = np.empty(g.shape, np.float32)
    _load().orc_silu_mul_array(_p(g), _p(u), g.size, _p(out))
    return out


def quantize_rows(x: np.ndarray):
    """(codes u8[rows][cols], scales f32[rows][cols/128]) for f32 x[rows][cols]."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    rows, cols = x.shape
    if cols % 128:
        raise ValueError("cols must be a multiple of 128")
    q = np.empty((rows, cols), np.uint8)
    s = np.empty((rows, cols // 128), np.float32)
    _load().orc_quantize_rows(_p(x), rows, cols, _p(q), _p(s))
    return q, s


def plan(ids: np.ndarray, E: int):
    """Stable counting sort of the slots by expert: (counts, offsets, perm, inv, n_bad)."""
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    T, k = ids.shape
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    perm = np.empty(max(T * k, 1), np.int32)
    inv = np.empty(max(T * k, 1), np.int32)
    bad = _load().orc_plan(_p(ids), T, k, E, _p(counts), _p(offsets), _p(perm), _p(inv))
    return counts, offsets, perm[: offsets[E]], inv[: T * k], int(bad)


def route(logits: np.ndarray, k: int, kind: int):
    """Top-k router on FP32 logits [T][E]: (ids int32[T][k] in descending
    logit order, ties to the lower id, NaN last; weights float64[T][k],
    softmax (kind 0) or sigmoid (kind 1) scores normalised over the chosen)."""
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = logits.shape
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    if _load().orc_route(_p(logits), T, E, k, kind, _p(ids), _p(w)) != 0:
        raise ValueError("bad router arguments")
    return ids, w


def slice_matrix(codes: np.ndarray, scales: np.ndarray, axis: int, off: int, length: int):
    """Slice one [R][C] code matrix (block scales [ceil(R/128)][ceil(C/128)])
    along rows (axis 0) or columns (axis 1) to [off, off+length), with the
    load-time requant when off is not a multiple of 128."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.float32)
    R, C = codes.shape
    oR, oC = (length, C) if axis == 0 else (R, length)
    oc = np.empty((oR, oC), np.uint8)
    os_ = np.empty(((oR + 127) // 128, (oC + 127) // 128), np.float32)
    if _load().orc_slice_matrix(_p(codes), _p(scales), R, C, axis, off, length, _p(oc), _p(os_)) != 0:
        raise ValueError("bad slice arguments")
    return oc, os_


def slice_layer(layer, off: int, inter: int):
    """The layer's experts restricted to intermediate features [off, off+inter)
    (gate / up rows, down columns), requantised when off % 128 != 0."""
    E = layer.gate.shape[0]
    out = {k: [] for k in ("gate", "up", "down", "gate_scale", "up_scale", "down_scale")}
    for e in range(E):
        for name, axis in (("gate", 0), ("up", 0), ("down", 1)):
            c, s = slice_matrix(getattr(layer, name)[e], getattr(layer, name + "_scale")[e], axis, off, inter)
            out[name].append(c)
            out[name + "_scale"].append(s)
    arrs = {k: np.stack(v) for k, v in out.items()}
    return type(layer)(layer.E, layer.H, inter, arrs["gate"], arrs["up"], arrs["down"],
                       arrs["gate_scale"], arrs["up_scale"], arrs["down_scale"])


def _layer_struct(layer):
    arrs = [np.ascontiguousarray(a) for a in (layer.gate, layer.up, layer.down)]
    sc = [np.ascontiguousarray(a, dtype=np.float32) for a in
          (layer.gate_scale, layer.up_scale, layer.down_scale)]
    st = _Layer(layer.E, layer.H, layer.I, *(a.ctypes.data for a in arrs),
                *(a.ctypes.data for a in sc))
    return st, arrs + sc  # keep the arrays alive


def forward(layer, x_bits: np.ndarray, ids: np.ndarray, w: np.ndarray, rho: float,
            out_dtype: int = OUT_BF16, debug: bool = False, n_shared: int = 0, a16: bool = False):
    """The layer on T tokens.  Returns out (u16 bf16 bits or f32 [T][H]) and,
    with debug=True, a dict of the intermediate arrays (sorted-order rows).
    n_shared: the last n_shared columns of ids / w are shared-expert slots,
    added outside rho.  a16: the W8A16 form (x and h stay 16-bit; debug then
    has hb, h as BF16 bits, instead of xq / sx / hq / sh)."""
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    w = np.ascontiguousarray(w, dtype=np.float32)
    T, k = ids.shape
    H, I, E = layer.H, layer.I, layer.E
    Ip = 128 * ((I + 127) // 128)
    out = np.empty((T, H), np.uint16 if out_dtype == OUT_BF16 else np.float32)
    st, keep = _layer_struct(layer)
    dbg = None
    d = None
    if debug:
        routed = int(((ids >= 0) & (ids < E)).sum())
        d = dict(xq=np.empty((T, H), np.uint8), sx=np.empty((T, H // 128), np.float32),
                 gu=np.empty((routed, 2 * Ip), np.float32), hq=np.empty((routed, Ip), np.uint8),
                 sh=np.empty((routed, Ip // 128), np.float32), y=np.empty((routed, H), np.float32),
                 counts=np.empty(E, np.int32), offsets=np.empty(E + 1, np.int32),
                 perm=np.empty(max(routed, 1), np.int32), inv=np.empty(max(T * k, 1), np.int32))
        if a16:
            d["hb"] = np.empty((routed, Ip), np.uint16)
            for n in ("xq", "sx", "hq", "sh"):
                del d[n]
        dbg = _Debug(*(d[n].ctypes.data if n in d else None for n in
                       ("xq", "sx", "gu", "hq", "sh", "y", "counts", "offsets", "perm", "inv", "hb")))
    fn = _load().orc_forward_a16 if a16 else _load().orc_forward
    bad = fn(ctypes.byref(st), k, _p(x_bits), _p(ids), _p(w), T, float(rho),
             out_dtype, _p(out), ctypes.byref(dbg) if dbg is not None else None, n_shared)
    del keep
    if bad < 0:
        raise ValueError("bad arguments")
    if debug:
        d["perm"] = d["perm"][: d["offsets"][E]]
        d["inv"] = d["inv"][: T * k]
        d["n_bad"] = int(bad)
        return out, d
    return out


def forward_a16(layer, x_bits, ids, w, rho, out_dtype: int = OUT_BF16, debug: bool = False,
                n_shared: int = 0):
    """The W8A16 form of forward (see orc_forward_a16 in oracle.c)."""
    return forward(layer, x_bits, ids, w, rho, out_dtype, debug, n_shared, a16=True)


def down_combine(layer, hq: np.ndarray, sh: np.ndarray, ids: np.ndarray, w: np.ndarray, rho: float,
                 out_dtype: int = OUT_BF16, n_shared: int = 0):
    """Continue the layer from given h codes (sorted order of the plan of ids).
    Returns (out, y)."""
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    w = np.ascontiguousarray(w, dtype=np.float32)
    hq = np.ascontiguousarray(hq, dtype=np.uint8)
    sh = np.ascontiguousarray(sh, dtype=np.float32)
    T, k = ids.shape
    out = np.empty((T, layer.H), np.uint16 if out_dtype == OUT_BF16 else np.float32)
    y = np.empty((max(hq.shape[0], 1), layer.H), np.float32)
    st, keep = _layer_struct(layer)
    P = _load().orc_down_combine(ctypes.byref(st), k, _p(hq), _p(sh), _p(ids), _p(w), T, float(rho),
                                 out_dtype, _p(out), _p(y), n_shared)
    del keep
    if P < 0 or P != hq.shape[0]:
        raise ValueError("bad arguments or h rows do not match the plan")
    return out, y[:P]


def bruteforce_fp64(layer, x_bits, ids, w, rho, quantize_activations=True, n_shared: int = 0) -> np.ndarray:
    """Dense FP64 evaluation (tiny inputs only).  out f64[T][H]."""
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    w = np.ascontiguousarray(w, dtype=np.float32)
    T, k = ids.shape
    out = np.empty((T, layer.H), np.float64)
    st, keep = _layer_struct(layer)
    _load().orc_bruteforce_fp64(ctypes.byref(st), k, _p(x_bits), _p(ids), _p(w), T, float(rho),
                                1 if quantize_activations else 0, _p(out), n_shared)
    del keep
    return out
