"""Routed-expert FP8 MoE prefill on MI355X: thin ctypes binding of the C ABI.

Every function here marshals arguments for the entry point of the same name in
``libmoe_fp8_prefill.so`` (declared in ``include/moe_fp8_prefill.h``); all
computation happens in the library's HIP kernels.  Device memory and streams
come from PyTorch (tensors' ``data_ptr()``, ``torch.cuda.current_stream()``).
There is no fallback: if the library is missing or does not load, every call
raises.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_fp8_prefill.so")

MOE_OK = 0
MOE_ERR_INVALID_ARG = 1
MOE_ERR_UNSUPPORTED = 2
MOE_ERR_OUT_OF_MEMORY = 3
MOE_ERR_DEVICE = 4
MOE_ERR_FAILED_STATE = 5
MOE_ERR_BUSY = 6
MOE_ERR_BAD_EXPERT_ID = 7

MOE_DTYPE_BF16 = 0
MOE_DTYPE_F32 = 1
MOE_ACT_SILU_UNCLAMPED = 0
MOE_ACT_SILU_CLAMPED = 1
MOE_ROUTER_SOFTMAX = 0
MOE_ROUTER_SIGMOID = 1
MOE_NUM_STAGES = 9
MOE_CALIBRATE_MFMA = 0
MOE_CALIBRATE_STREAM = 1
STAGES = ("plan", "quant", "gate_up_stream", "gate_up_narrow", "gate_up_wide", "down_stream", "down_narrow",
          "down_wide", "combine")

EXPORTED = (
    "moe_fp8_prefill_validate", "moe_fp8_prefill_workspace_bytes", "moe_fp8_prefill_weight_bytes",
    "moe_fp8_prefill_create", "moe_fp8_prefill_run", "moe_fp8_prefill_status",
    "moe_fp8_prefill_destroy", "moe_fp8_prefill_strerror", "moe_fp8_prefill_debug_plan",
    "moe_fp8_prefill_debug_activations", "moe_fp8_prefill_debug_intermediates",
    "moe_fp8_prefill_debug_gate_up",
    "moe_fp8_prefill_debug_unpack", "moe_fp8_prefill_debug_mfma", "moe_fp8_prefill_set_timing",
    "moe_fp8_prefill_set_timing_stages", "moe_fp8_prefill_read_timing", "moe_fp8_prefill_debug_inject_failure",
    "moe_fp8_prefill_route", "moe_fp8_prefill_run_logits", "moe_fp8_prefill_run_decode",
    "moe_fp8_prefill_create_streamed", "moe_fp8_prefill_stage", "moe_fp8_prefill_select_slot",
    "moe_fp8_prefill_calibrate", "moe_fp8_prefill_run_static",
)


class MoeError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {moe_fp8_prefill_strerror(code)} (code {code})")


class moe_fp8_prefill_desc(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_int32), ("num_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
        ("hidden", ctypes.c_int32), ("inter", ctypes.c_int32), ("max_rows", ctypes.c_int32),
        ("out_dtype", ctypes.c_int32), ("activation", ctypes.c_int32), ("block", ctypes.c_int32),
        ("routed_scale", ctypes.c_float), ("weights_on_device", ctypes.c_int32),
        ("gate", ctypes.c_void_p), ("up", ctypes.c_void_p), ("down", ctypes.c_void_p),
        ("gate_scale", ctypes.c_void_p), ("up_scale", ctypes.c_void_p), ("down_scale", ctypes.c_void_p),
        ("stream", ctypes.c_void_p), ("shared_experts", ctypes.c_int32),
        ("activation_limit", ctypes.c_float), ("inter_full", ctypes.c_int32),
        ("inter_offset", ctypes.c_int32),
    ]


_lib = None


def load_library() -> ctypes.CDLL:
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with fp8_blockwise_routed_amd/build.py")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    D = ctypes.POINTER(moe_fp8_prefill_desc)
    sig = {
        "moe_fp8_prefill_validate": ([D], ctypes.c_int),
        "moe_fp8_prefill_workspace_bytes": ([D], I64),
        "moe_fp8_prefill_weight_bytes": ([D], I64),
        "moe_fp8_prefill_create": ([D, ctypes.POINTER(P)], ctypes.c_int),
        "moe_fp8_prefill_run": ([P, P, P, P, I64, P, P], ctypes.c_int),
        "moe_fp8_prefill_run_decode": ([P, P, P, P, I64, P, P], ctypes.c_int),
        "moe_fp8_prefill_run_static": ([P, P, P, P, I64, P, P], ctypes.c_int),
        "moe_fp8_prefill_status": ([P], ctypes.c_int),
        "moe_fp8_prefill_destroy": ([P], None),
        "moe_fp8_prefill_strerror": ([ctypes.c_int], ctypes.c_char_p),
        "moe_fp8_prefill_debug_plan": ([P, P, P, P, P, I64], ctypes.c_int),
        "moe_fp8_prefill_debug_activations": ([P, P, P, I64], ctypes.c_int),
        "moe_fp8_prefill_debug_intermediates": ([P, P, P, P, I64, ctypes.POINTER(I64)], ctypes.c_int),
        "moe_fp8_prefill_debug_gate_up": ([P, P, I64, ctypes.POINTER(I64)], ctypes.c_int),
        "moe_fp8_prefill_debug_unpack": ([P, I32, P, P, P, P, P, P], ctypes.c_int),
        "moe_fp8_prefill_debug_mfma": ([P, P, P], ctypes.c_int),
        "moe_fp8_prefill_set_timing": ([P, I32], ctypes.c_int),
        "moe_fp8_prefill_set_timing_stages": ([P, ctypes.c_uint32], ctypes.c_int),
        "moe_fp8_prefill_read_timing": ([P, P, I32, ctypes.POINTER(I32)], ctypes.c_int),
        "moe_fp8_prefill_debug_inject_failure": ([P], ctypes.c_int),
        "moe_fp8_prefill_route": ([P, P, I32, I64, P, P, P], ctypes.c_int),
        "moe_fp8_prefill_run_logits": ([P, P, P, I32, I64, P, P], ctypes.c_int),
        "moe_fp8_prefill_create_streamed": ([D, I32, ctypes.POINTER(P)], ctypes.c_int),
        "moe_fp8_prefill_stage": ([P, I32, P, P, P, P, P, P, P], ctypes.c_int),
        "moe_fp8_prefill_select_slot": ([P, I32], ctypes.c_int),
        "moe_fp8_prefill_calibrate": ([I32, I64, P, I64, P, ctypes.POINTER(ctypes.c_double)], ctypes.c_int),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def _np_ptr(a):
    if a is None:
        return None
    if not (isinstance(a, np.ndarray) and a.flags["C_CONTIGUOUS"]):
        raise ValueError("need a C-contiguous numpy array")
    return ctypes.c_void_p(a.ctypes.data)


def _dev_ptr(t):
    """Device pointer of a torch CUDA tensor (or an int address)."""
    if t is None:
        return None
    if isinstance(t, int):
        return ctypes.c_void_p(t)
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError("need a contiguous device tensor")
    return ctypes.c_void_p(t.data_ptr())


def _stream_ptr(stream):
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _check(rc: int, where: str) -> None:
    if rc != MOE_OK:
        raise MoeError(rc, where)


# ---- the C ABI, one wrapper per entry point --------------------------------

def make_desc(layer, top_k: int, max_rows: int = 8192, out_dtype: int = MOE_DTYPE_BF16,
              routed_scale: float = 1.0, activation: int = MOE_ACT_SILU_UNCLAMPED,
              block: int = 128, stream=None, on_device: bool = False, shared_experts: int = 0,
              activation_limit: float = 0.0, share=None):
    """Description for a layer held as numpy arrays (or, with on_device=True,
    torch device tensors) with fields gate, up, down, gate_scale, up_scale,
    down_scale, E, H, I.  With shared_experts=1 the arrays hold layer.E
    experts, the last one shared (E - 1 routed).  Keep the returned arrays
    alive until create().  share=(offset, length): use intermediate features
    [offset, offset + length) of the arrays' layer.I."""
    arrs = [layer.gate, layer.up, layer.down, layer.gate_scale, layer.up_scale, layer.down_scale]
    if on_device:
        ptrs = [a.data_ptr() for a in arrs]
    else:
        arrs = [np.ascontiguousarray(a) for a in arrs]
        ptrs = [a.ctypes.data for a in arrs]
    inter, i_full, i_off = layer.I, 0, 0
    if share is not None:
        i_off, inter = share
        i_full = layer.I
    d = moe_fp8_prefill_desc(ctypes.sizeof(moe_fp8_prefill_desc), layer.E - shared_experts, top_k,
                             layer.H, inter, max_rows, out_dtype, activation, block, routed_scale,
                             1 if on_device else 0, *ptrs,
                             None if stream is None else _stream_ptr(stream).value, shared_experts,
                             activation_limit, i_full, i_off)
    return d, arrs


def moe_fp8_prefill_validate(desc) -> int:
    return int(load_library().moe_fp8_prefill_validate(ctypes.byref(desc)))


def moe_fp8_prefill_workspace_bytes(desc) -> int:
    return int(load_library().moe_fp8_prefill_workspace_bytes(ctypes.byref(desc)))


def moe_fp8_prefill_weight_bytes(desc) -> int:
    return int(load_library().moe_fp8_prefill_weight_bytes(ctypes.byref(desc)))


def moe_fp8_prefill_create(desc) -> int:
    """Returns the handle (an opaque address); raises MoeError."""
    h = ctypes.c_void_p()
    _check(load_library().moe_fp8_prefill_create(ctypes.byref(desc), ctypes.byref(h)),
           "moe_fp8_prefill_create")
    return h.value


def moe_fp8_prefill_run(handle: int, x, ids, w, T: int, out, stream=None) -> int:
    """Returns the MOE_* code (does not raise) so callers can test error paths."""
    return int(load_library().moe_fp8_prefill_run(ctypes.c_void_p(handle), _dev_ptr(x), _dev_ptr(ids),
                                                  _dev_ptr(w), T, _dev_ptr(out), _stream_ptr(stream)))


def moe_fp8_prefill_run_decode(handle: int, x, ids, w, T: int, out, stream=None) -> int:
    """The W8A16 decode path; returns the MOE_* code."""
    return int(load_library().moe_fp8_prefill_run_decode(ctypes.c_void_p(handle), _dev_ptr(x), _dev_ptr(ids),
                                                         _dev_ptr(w), T, _dev_ptr(out), _stream_ptr(stream)))


def moe_fp8_prefill_run_static(handle: int, x, ids, w, T: int, out, stream=None) -> int:
    """run() with its per-pass workspace in the library's static device array
    (allocates nothing); returns the MOE_* code."""
    return int(load_library().moe_fp8_prefill_run_static(ctypes.c_void_p(handle), _dev_ptr(x), _dev_ptr(ids),
                                                         _dev_ptr(w), T, _dev_ptr(out), _stream_ptr(stream)))


def moe_fp8_prefill_route(handle: int, logits, router: int, T: int, ids, w, stream=None) -> int:
    """Returns the MOE_* code."""
    return int(load_library().moe_fp8_prefill_route(ctypes.c_void_p(handle), _dev_ptr(logits), router, T,
                                                    _dev_ptr(ids), _dev_ptr(w), _stream_ptr(stream)))


def moe_fp8_prefill_run_logits(handle: int, x, logits, router: int, T: int, out, stream=None) -> int:
    """Returns the MOE_* code."""
    return int(load_library().moe_fp8_prefill_run_logits(ctypes.c_void_p(handle), _dev_ptr(x),
                                                         _dev_ptr(logits), router, T, _dev_ptr(out),
                                                         _stream_ptr(stream)))


def _host_ptr(a):
    """Host address of a C-contiguous numpy array or a contiguous CPU torch
    tensor (pinned or not)."""
    if isinstance(a, np.ndarray):
        return _np_ptr(a)
    if a.is_cuda or not a.is_contiguous():
        raise ValueError("need a contiguous host tensor")
    return ctypes.c_void_p(a.data_ptr())


def moe_fp8_prefill_create_streamed(desc, n_slots: int) -> int:
    """Returns the handle of a streamed-slot layer (no weights uploaded)."""
    h = ctypes.c_void_p()
    _check(load_library().moe_fp8_prefill_create_streamed(ctypes.byref(desc), n_slots, ctypes.byref(h)),
           "moe_fp8_prefill_create_streamed")
    return h.value


def moe_fp8_prefill_stage(handle: int, slot: int, gate, up, down, gate_scale, up_scale, down_scale,
                          stream=None) -> int:
    """Returns the MOE_* code.  Arrays: numpy or (pinned) CPU torch tensors in
    the canonical layout; they must stay alive until the stream passes."""
    return int(load_library().moe_fp8_prefill_stage(
        ctypes.c_void_p(handle), slot, _host_ptr(gate), _host_ptr(up), _host_ptr(down),
        _host_ptr(gate_scale), _host_ptr(up_scale), _host_ptr(down_scale), _stream_ptr(stream)))


def moe_fp8_prefill_select_slot(handle: int, slot: int) -> int:
    return int(load_library().moe_fp8_prefill_select_slot(ctypes.c_void_p(handle), slot))


def moe_fp8_prefill_status(handle: int) -> int:
    return int(load_library().moe_fp8_prefill_status(ctypes.c_void_p(handle)))


def moe_fp8_prefill_destroy(handle) -> None:
    load_library().moe_fp8_prefill_destroy(ctypes.c_void_p(handle) if handle else None)


def moe_fp8_prefill_strerror(code: int) -> str:
    return load_library().moe_fp8_prefill_strerror(code).decode()


def moe_fp8_prefill_debug_plan(handle: int, E: int, n_slots: int):
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    perm = np.empty(max(n_slots, 1), np.int32)
    inv = np.empty(max(n_slots, 1), np.int32)
    _check(load_library().moe_fp8_prefill_debug_plan(ctypes.c_void_p(handle), _np_ptr(counts),
                                                     _np_ptr(offsets), _np_ptr(perm), _np_ptr(inv),
                                                     n_slots), "moe_fp8_prefill_debug_plan")
    return counts, offsets, perm[: offsets[E]], inv[:n_slots]


def moe_fp8_prefill_debug_activations(handle: int, rows: int, H: int):
    xq = np.empty((rows, H), np.uint8)
    sx = np.empty((rows, H // 128), np.float32)
    _check(load_library().moe_fp8_prefill_debug_activations(ctypes.c_void_p(handle), _np_ptr(xq),
                                                            _np_ptr(sx), rows),
           "moe_fp8_prefill_debug_activations")
    return xq, sx


def moe_fp8_prefill_debug_intermediates(handle: int, cap_rows: int, H: int, Ip: int):
    hq = np.empty((cap_rows, Ip), np.uint8)
    sh = np.empty((cap_rows, Ip // 128), np.float32)
    y = np.empty((cap_rows, H), np.float32)
    n = ctypes.c_int64()
    _check(load_library().moe_fp8_prefill_debug_intermediates(ctypes.c_void_p(handle), _np_ptr(hq),
                                                              _np_ptr(sh), _np_ptr(y), cap_rows,
                                                              ctypes.byref(n)),
           "moe_fp8_prefill_debug_intermediates")
    return hq[: n.value], sh[: n.value], y[: n.value]


def moe_fp8_prefill_debug_gate_up(handle: int, cap_rows: int, Ip: int):
    gu = np.empty((max(cap_rows, 1), 2 * Ip), np.float32)
    n = ctypes.c_int64()
    _check(load_library().moe_fp8_prefill_debug_gate_up(ctypes.c_void_p(handle), _np_ptr(gu), cap_rows,
                                                        ctypes.byref(n)),
           "moe_fp8_prefill_debug_gate_up")
    return gu[: n.value]


def moe_fp8_prefill_debug_unpack(handle: int, e: int, H: int, I: int):
    nI, nH = (I + 127) // 128, H // 128
    out = dict(gate=np.empty((I, H), np.uint8), up=np.empty((I, H), np.uint8),
               down=np.empty((H, I), np.uint8), gate_scale=np.empty((nI, nH), np.float32),
               up_scale=np.empty((nI, nH), np.float32), down_scale=np.empty((nH, nI), np.float32))
    _check(load_library().moe_fp8_prefill_debug_unpack(
        ctypes.c_void_p(handle), e, *(_np_ptr(out[k]) for k in
                                      ("gate", "up", "down", "gate_scale", "up_scale", "down_scale"))),
        "moe_fp8_prefill_debug_unpack")
    return out


def moe_fp8_prefill_debug_mfma(a: np.ndarray, b: np.ndarray, both: bool = False) -> np.ndarray:
    a = np.ascontiguousarray(a, np.uint8).reshape(16, 128)
    b = np.ascontiguousarray(b, np.uint8).reshape(16, 128)
    d = np.empty((3, 16, 16), np.float32)
    _check(load_library().moe_fp8_prefill_debug_mfma(_np_ptr(a), _np_ptr(b), _np_ptr(d)),
           "moe_fp8_prefill_debug_mfma")
    return d[0] if not both else d


def moe_fp8_prefill_calibrate(kind: int, n: int, buf, stream=None) -> float:
    """Enqueue a calibration launch on `stream` over the device tensor buf;
    returns its algorithmic work (FLOPs or bytes)."""
    work = ctypes.c_double(0.0)
    nbytes = int(buf.numel() * buf.element_size())
    _check(load_library().moe_fp8_prefill_calibrate(int(kind), int(n), _dev_ptr(buf), nbytes,
                                                   _stream_ptr(stream), ctypes.byref(work)), "calibrate")
    return work.value


def moe_fp8_prefill_set_timing(handle: int, enable: bool) -> None:
    _check(load_library().moe_fp8_prefill_set_timing(ctypes.c_void_p(handle), 1 if enable else 0),
           "moe_fp8_prefill_set_timing")


def moe_fp8_prefill_set_timing_stages(handle: int, stages) -> None:
    """Time only the named stages (names from STAGES); an empty list turns timing off."""
    mask = 0
    for name in stages:
        mask |= 1 << STAGES.index(name)
    _check(load_library().moe_fp8_prefill_set_timing_stages(ctypes.c_void_p(handle), mask),
           "moe_fp8_prefill_set_timing_stages")


def moe_fp8_prefill_read_timing(handle: int, max_records: int = 4096) -> np.ndarray:
    """[records][MOE_NUM_STAGES] milliseconds, one row per pass, in the order of STAGES
    (-1 for a stage that was not timed)."""
    buf = np.zeros((max_records, MOE_NUM_STAGES), np.float32)
    n = ctypes.c_int32()
    _check(load_library().moe_fp8_prefill_read_timing(ctypes.c_void_p(handle), _np_ptr(buf),
                                                      max_records, ctypes.byref(n)),
           "moe_fp8_prefill_read_timing")
    return buf[: n.value]


def moe_fp8_prefill_debug_inject_failure(handle: int) -> None:
    _check(load_library().moe_fp8_prefill_debug_inject_failure(ctypes.c_void_p(handle)),
           "moe_fp8_prefill_debug_inject_failure")


# ---- convenience wrappers --------------------------------------------------

class MoeFp8Prefill:
    """Owns one handle.  ``layer`` has numpy fields gate, up, down, gate_scale,
    up_scale, down_scale and E, H, I (the canonical checkpoint layout)."""

    def __init__(self, layer, top_k: int, routed_scale: float = 1.0, max_rows: int = 8192,
                 out_dtype: int = MOE_DTYPE_BF16, on_device: bool = False, shared_experts: int = 0,
                 activation_limit: float = 0.0, share=None):
        """activation_limit > 0 selects the clamped SiLU with that limit;
        share=(offset, length) takes intermediate features [offset,
        offset + length) of the layer (requantised at load if unaligned)."""
        # E, k: routed experts and slots; the shared expert is the arrays' last
        self.E, self.H, self.I, self.k = layer.E - shared_experts, layer.H, layer.I, top_k
        if share is not None:
            self.I = share[1]
        self.shared = shared_experts
        self.Ip = 128 * ((self.I + 127) // 128)
        self.out_dtype = out_dtype
        self.max_rows = max_rows
        act = MOE_ACT_SILU_CLAMPED if activation_limit > 0 else MOE_ACT_SILU_UNCLAMPED
        desc, keep = make_desc(layer, top_k, max_rows, out_dtype, routed_scale, activation=act,
                               on_device=on_device, shared_experts=shared_experts,
                               activation_limit=activation_limit, share=share)
        self.handle = moe_fp8_prefill_create(desc)
        del keep

    def run(self, x, ids, w, out=None, stream=None):
        """x: bf16 [T][H], ids: int32 [T][k], w: float32 [T][k] (torch device tensors)."""
        import torch
        T = x.shape[0]
        if out is None:
            dt = torch.float32 if self.out_dtype == MOE_DTYPE_F32 else torch.bfloat16
            out = torch.empty((T, self.H), dtype=dt, device=x.device)
        _check(moe_fp8_prefill_run(self.handle, x, ids, w, T, out, stream), "moe_fp8_prefill_run")
        return out

    def run_decode(self, x, ids, w, out=None, stream=None):
        """The W8A16 decode path (x and h stay 16-bit); arguments as run()."""
        import torch
        T = x.shape[0]
        if out is None:
            dt = torch.float32 if self.out_dtype == MOE_DTYPE_F32 else torch.bfloat16
            out = torch.empty((T, self.H), dtype=dt, device=x.device)
        _check(moe_fp8_prefill_run_decode(self.handle, x, ids, w, T, out, stream), "moe_fp8_prefill_run_decode")
        return out

    def route(self, logits, router: int, stream=None):
        """logits: float32 [T][E] device tensor -> (ids int32 [T][k], w float32 [T][k])."""
        import torch
        T = logits.shape[0]
        ids = torch.empty((T, self.k), dtype=torch.int32, device=logits.device)
        w = torch.empty((T, self.k), dtype=torch.float32, device=logits.device)
        _check(moe_fp8_prefill_route(self.handle, logits, router, T, ids, w, stream), "moe_fp8_prefill_route")
        return ids, w

    def run_logits(self, x, logits, router: int, out=None, stream=None):
        """x: bf16 [T][H], logits: float32 [T][E] (torch device tensors)."""
        import torch
        T = x.shape[0]
        if out is None:
            dt = torch.float32 if self.out_dtype == MOE_DTYPE_F32 else torch.bfloat16
            out = torch.empty((T, self.H), dtype=dt, device=x.device)
        _check(moe_fp8_prefill_run_logits(self.handle, x, logits, router, T, out, stream),
               "moe_fp8_prefill_run_logits")
        return out

    def status(self) -> int:
        return moe_fp8_prefill_status(self.handle)

    def close(self) -> None:
        if self.handle:
            moe_fp8_prefill_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class StreamedMoeFp8Prefill(MoeFp8Prefill):
    """A layer handle with n_slots device weight slots that the caller fills
    layer by layer with stage() (host arrays in the canonical layout) and
    picks with select().  ``shape`` has E, H, I (E counting a shared expert)."""

    def __init__(self, shape, top_k: int, n_slots: int = 2, routed_scale: float = 1.0,
                 max_rows: int = 8192, out_dtype: int = MOE_DTYPE_BF16, shared_experts: int = 0,
                 activation_limit: float = 0.0, share=None):
        self.E, self.H, self.I, self.k = shape.E - shared_experts, shape.H, shape.I, top_k
        inter, i_full, i_off = shape.I, 0, 0
        if share is not None:
            i_off, inter = share
            i_full = shape.I
            self.I = inter
        self.Ip = 128 * ((self.I + 127) // 128)
        self.out_dtype = out_dtype
        self.max_rows = max_rows
        self.shared = shared_experts
        act = MOE_ACT_SILU_CLAMPED if activation_limit > 0 else MOE_ACT_SILU_UNCLAMPED
        desc = moe_fp8_prefill_desc(ctypes.sizeof(moe_fp8_prefill_desc), shape.E - shared_experts, top_k,
                                    shape.H, inter, max_rows, out_dtype, act, 128, routed_scale, 0,
                                    None, None, None, None, None, None, None, shared_experts,
                                    activation_limit, i_full, i_off)
        self.handle = moe_fp8_prefill_create_streamed(desc, n_slots)

    def stage(self, slot: int, layer, stream=None) -> None:
        _check(moe_fp8_prefill_stage(self.handle, slot, layer.gate, layer.up, layer.down, layer.gate_scale,
                                     layer.up_scale, layer.down_scale, stream), "moe_fp8_prefill_stage")

    def select(self, slot: int) -> None:
        _check(moe_fp8_prefill_select_slot(self.handle, slot), "moe_fp8_prefill_select_slot")
