"""Pins of the CPU oracle against facts other than itself.

Each pin returns (ok, detail).  The tests assert them; test_oracle_faults.py
plants mistakes in the oracle and checks that some pin turns red.

What pins what:
  decode     golden values printed by the pages (tests/golden/e4m3_decode.txt),
             torch's float8_e4m3fn widening (a library routine), and structure
             (sign symmetry, monotonicity, subnormal step).
  encode     torch's float8_e4m3fn narrowing (RNE) on a reduced-exhaustive set
             of FP32 patterns; an exhaustive nearest-code search; round trip;
             saturation and specials.
  bf16       torch's bfloat16 conversions, exhaustive / midpoints.
  quantiser  a torch re-derivation (amax, IEEE divide, torch float8 cast) and
             invariants (amax element -> +-448, error bounds).
  plan       numpy's stable argsort.
  router     a sort by (logit descending, id ascending) in plain Python with
             NaN last; scipy's full softmax renormalised over the chosen
             experts and scipy's expit; the generator's own FP64 top-k on the
             same draws; tie, -inf, NaN and k = E cases; shift invariance of
             the softmax weights.
  shared     the FP64 brute force with the shared slot outside rho; the
             routed layer plus the shared expert evaluated on its own.
  clamp      the FP64 brute force with the clamped SwiGLU; h from the
             oracle's own gate/up through a numpy clamp; a limit above every
             |gate|, |up| reproduces the unclamped bits.
  slice      an aligned slice = numpy slicing of codes and scales; the
             requant of an unaligned slice = a torch re-derivation (FP32
             dequantise, block amax / 448, float8 cast) bit for bit, within
             the E4M3 rounding bound of the checkpoint values; two slices'
             FP64 brute forces add up to the full layer's.
  layer      the FP64 dense brute force (different loop structure, FP64,
             exhaustive-search encoder); a dense gated FFN evaluated with torch
             float8 casts and float64 matmuls; an integer-exact case compared
             bit for bit with int64 matmuls; linearity, permutation, skip-slot
             and NaN-isolation properties; the down stage against a float64
             matmul of its dequantised operands.
"""
from __future__ import annotations

import os

import numpy as np
import torch

import gen
import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _ok(cond, detail=""):
    return (bool(cond), detail)


# ---------------------------------------------------------------- codecs ---

def read_golden_decode():
    rows = []
    with open(os.path.join(GOLDEN, "e4m3_decode.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = line.split()
            rows.append((int(parts[0], 16), float(parts[1])))
    return rows


def pin_decode_golden():
    rows = read_golden_decode()
    codes = np.array([c for c, _ in rows], np.uint8)
    got = oracle.e4m3_decode(codes)
    exp = np.array([v for _, v in rows], np.float32)
    bad = [(hex(c), float(g), float(e)) for c, g, e in zip(codes, got, exp)
           if g.view(np.uint32) != e.view(np.uint32)]
    return _ok(not bad, f"mismatches {bad[:5]}")


def pin_decode_vs_torch():
    codes = np.arange(256, dtype=np.uint8)
    got = oracle.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    finite = ~np.isnan(ref)  # torch widens the two NaN codes to NaN
    bad = np.nonzero(got[finite].view(np.uint32) != ref[finite].view(np.uint32))[0]
    return _ok(finite.sum() == 254 and bad.size == 0, f"{bad.size} mismatches")


def pin_decode_structure():
    v = oracle.e4m3_decode(np.arange(256, dtype=np.uint8))
    pos, neg = v[:128], v[128:]
    sym = np.all((-pos).view(np.uint32) == neg.view(np.uint32))
    mono = np.all(np.diff(pos[:127].astype(np.float64)) > 0)
    sub = np.all(pos[:8] == np.arange(8, dtype=np.float32) * np.float32(2.0 ** -9))
    nan_zero = v[0x7F] == 0 and not np.signbit(v[0x7F]) and v[0xFF] == 0 and np.signbit(v[0xFF])
    return _ok(sym and mono and sub and nan_zero, f"sym={sym} mono={mono} sub={sub} nan0={nan_zero}")


def reduced_exhaustive_f32(limit_abs=463.9):
    """All (sign, exponent, top-11 mantissa bits) FP32 patterns combined with
    low-12-bit patterns that cover exact ties and their neighbours."""
    hi = np.arange(1 << 20, dtype=np.uint32) << 12
    lows = np.array([0x000, 0x001, 0x7FF, 0x800, 0x801, 0xFFF], np.uint32)
    bits = (hi[:, None] | lows[None, :]).ravel()
    v = bits.view(np.float32)
    keep = np.isfinite(v) & (np.abs(v) <= limit_abs)
    return v[keep]


def pin_encode_vs_torch(sample=None):
    v = reduced_exhaustive_f32() if sample is None else sample
    got = oracle.e4m3_encode(v)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    bad = np.nonzero(got != ref)[0]
    detail = "" if bad.size == 0 else f"{bad.size} mismatches, e.g. {v[bad[:3]]} -> {got[bad[:3]]} vs {ref[bad[:3]]}"
    return _ok(bad.size == 0, detail)


def pin_encode_specials():
    cases = [(448.0, 0x7E), (463.99, 0x7E), (464.0, 0x7E), (1e6, 0x7E), (np.inf, 0x7E),
             (-np.inf, 0xFE), (-500.0, 0xFE), (0.0, 0x00), (-0.0, 0x80), (2.0 ** -11, 0x00),
             (-(2.0 ** -11), 0x80), (3 * 2.0 ** -11, 0x01), (np.nan, 0x00)]
    v = np.array([c[0] for c in cases], np.float32)
    got = oracle.e4m3_encode(v)
    exp = np.array([c[1] for c in cases], np.uint8)
    return _ok(np.array_equal(got, exp), f"{list(zip(v, got, exp))}")


def pin_encode_roundtrip():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    back = oracle.e4m3_encode(oracle.e4m3_decode(codes))
    return _ok(np.array_equal(back, codes), f"{np.nonzero(back != codes)[0][:5]}")


def pin_encode_vs_nearest_search(n=200000, seed=1):
    rng = np.random.default_rng(seed)
    mags = np.concatenate([rng.uniform(0, 500, n // 2),
                           np.exp2(rng.uniform(-12, 9, n // 2))]).astype(np.float32)
    v = np.where(rng.random(mags.size) < 0.5, -mags, mags).astype(np.float32)
    table = oracle.e4m3_decode(np.arange(0x7F, dtype=np.uint8)).astype(np.float64)
    got = oracle.e4m3_encode(v)
    a = np.abs(v.astype(np.float64))
    ok = True
    for lo in range(0, v.size, 20000):
        d = np.abs(a[lo:lo + 20000, None] - table[None, :])
        dmin = d.min(axis=1, keepdims=True)
        cand = d == dmin
        # ties go to the even code
        even_tie = cand & ((np.arange(0x7F)[None, :] & 1) == 0)
        pick = np.where(even_tie.any(axis=1), even_tie.argmax(axis=1), cand.argmax(axis=1))
        ref = pick.astype(np.uint8) | np.where(np.signbit(v[lo:lo + 20000]), 0x80, 0).astype(np.uint8)
        if not np.array_equal(ref, got[lo:lo + 20000]):
            ok = False
    return _ok(ok, "nearest-code search disagrees")


def pin_bf16_widen_vs_torch():
    b = np.arange(1 << 16, dtype=np.uint16)
    got = oracle.bf16_to_f32(b)
    ref = torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).float().numpy()
    same = (got.view(np.uint32) == ref.view(np.uint32)) | (np.isnan(got) & np.isnan(ref))
    return _ok(same.all(), f"{(~same).sum()} mismatches")


def pin_bf16_narrow_vs_torch(n=1 << 20, seed=2):
    rng = np.random.default_rng(seed)
    bits = rng.integers(0, 1 << 32, n, dtype=np.uint64).astype(np.uint32)
    # add exact midpoints (low 16 bits = 0x8000) and their neighbours
    mids = (bits[: n // 4] & 0xFFFF0000) | 0x8000
    bits = np.concatenate([bits, mids, mids + 1, mids - 1])
    v = bits.view(np.float32)
    v = v[np.isfinite(v)]
    got = oracle.f32_to_bf16(v)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return _ok(np.array_equal(got, ref), f"{(got != ref).sum()} mismatches")


# ------------------------------------------------------------- quantiser ---

def quant_test_rows(seed=3):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((16, 512)).astype(np.float32)
    x[1] *= 100.0                      # outlier row
    x[2, :128] = 0.0                   # all-zero group
    x[3, 128:256] *= 1e-6              # tiny group (subnormal codes)
    x[4, 256:384] = -0.0               # negative zeros
    x[5, 7] = 3e4                      # single spike
    x[6, :] = np.round(x[6, :] * 8) / 8
    return x


def pin_quantize_vs_torch():
    x = quant_test_rows()
    q, s = oracle.quantize_rows(x)
    g = torch.from_numpy(x).view(x.shape[0], -1, 128)
    amax = g.abs().amax(dim=-1)
    s_ref = amax / 448.0
    codes = (g / s_ref.clamp_min(torch.finfo(torch.float32).tiny)[..., None]).to(torch.float8_e4m3fn)
    codes = codes.view(torch.uint8).reshape(x.shape).numpy().copy()
    zero = (amax == 0).numpy()
    codes.reshape(x.shape[0], -1, 128)[zero] = 0
    ok_s = np.array_equal(s.view(np.uint32), s_ref.numpy().view(np.uint32))
    ok_q = np.array_equal(q, codes)
    return _ok(ok_s and ok_q, f"scales equal={ok_s} codes equal={ok_q}")


def pin_quantize_invariants():
    x = quant_test_rows()
    q, s = oracle.quantize_rows(x)
    dec = oracle.e4m3_decode(q).astype(np.float64)
    ok = True
    for r in range(x.shape[0]):
        for g in range(x.shape[1] // 128):
            xv = x[r, g * 128:(g + 1) * 128].astype(np.float64)
            qv = q[r, g * 128:(g + 1) * 128]
            sc = float(s[r, g])
            amax = np.abs(xv).max()
            if amax == 0:
                ok &= sc == 0 and np.all(qv == 0)
                continue
            i = int(np.argmax(np.abs(xv)))
            ok &= (qv[i] & 0x7F) == 0x7E
            err = np.abs(xv - sc * dec[r, g * 128:(g + 1) * 128])
            bound = np.maximum(np.abs(xv) * 2.0 ** -4, sc * 2.0 ** -10 * 1.0001)
            ok &= bool(np.all(err <= bound + 1e-30))
    return _ok(ok, "quantiser invariant violated")


# ------------------------------------------------------------------ plan ---

def plan_ids(seed=4):
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, 13, (97, 5)).astype(np.int32)
    ids[3, 2] = -1          # skip slot
    ids[10, :] = -1
    ids[20, 0] = 13         # bad id (>= E)
    ids[21, 4] = 999
    return ids, 13


def pin_plan_vs_numpy():
    ids, E = plan_ids()
    counts, offsets, perm, inv, bad = oracle.plan(ids, E)
    flat = ids.ravel()
    valid = (flat >= 0) & (flat < E)
    f = np.nonzero(valid)[0]
    order = f[np.argsort(flat[f], kind="stable")]
    c_ref = np.bincount(flat[valid], minlength=E)
    o_ref = np.concatenate([[0], np.cumsum(c_ref)])
    inv_ref = np.full(flat.size, -1, np.int64)
    inv_ref[order] = np.arange(order.size)
    ok = (np.array_equal(counts, c_ref) and np.array_equal(offsets, o_ref)
          and np.array_equal(perm, order) and np.array_equal(inv, inv_ref) and bad == 2)
    return _ok(ok, "plan differs from numpy stable argsort")


# ---------------------------------------------------------------- router ---

def router_logits(seed=9):
    rng = np.random.default_rng(seed)
    l = rng.standard_normal((64, 23)).astype(np.float32)
    l[3, [2, 7, 11]] = 1.5                    # three-way tie
    l[4, :] = 0.25                            # all equal
    l[5, [0, 1]] = -np.inf                    # masked experts
    l[6, 4] = np.nan                          # a NaN logit ranks last
    l[7, :] = -np.inf                         # no mass at all
    l[8, 5] = np.inf
    return l


def _sorted_topk(row, k):
    key = [((1, 0.0) if np.isnan(v) else (0, -float(v)), e) for e, v in enumerate(row)]
    return [e for _, e in sorted(key)[:k]]


def pin_route_ids_vs_sort():
    l = router_logits()
    ok = True
    for kind in (oracle.ROUTE_SOFTMAX, oracle.ROUTE_SIGMOID):
        for k in (1, 4, 8, l.shape[1]):
            ids, _ = oracle.route(l, k, kind)
            ref = np.array([_sorted_topk(r, k) for r in l], np.int32)
            ok &= np.array_equal(ids, ref)
    return _ok(ok, "router ids differ from a (logit desc, id asc) sort")


def pin_route_weights_vs_scipy():
    from scipy.special import expit, softmax
    l = router_logits()
    good = np.isfinite(l).all(axis=1)
    ok = True
    for k in (2, 8):
        ids, w = oracle.route(l, k, oracle.ROUTE_SOFTMAX)
        full = softmax(l[good].astype(np.float64), axis=1)
        ch = np.take_along_axis(full, ids[good].astype(np.int64), axis=1)
        ok &= np.allclose(w[good], ch / ch.sum(axis=1, keepdims=True), rtol=1e-12, atol=1e-15)
        ids, w = oracle.route(l, k, oracle.ROUTE_SIGMOID)
        sg = expit(np.take_along_axis(l[good].astype(np.float64), ids[good].astype(np.int64), axis=1))
        ok &= np.allclose(w[good], sg / sg.sum(axis=1, keepdims=True), rtol=1e-12, atol=1e-15)
    return _ok(ok, "router weights differ from scipy softmax / expit")


def pin_route_special_rows():
    l = router_logits()
    ok = True
    for kind in (oracle.ROUTE_SOFTMAX, oracle.ROUTE_SIGMOID):
        ids, w = oracle.route(l, 4, kind)
        full, _ = oracle.route(l[3:4], l.shape[1], kind)           # three-way tie
        pos = [list(full[0]).index(e) for e in (2, 7, 11)]
        ok &= pos == sorted(pos) and pos[2] - pos[0] == 2
        ok &= list(ids[4]) == [0, 1, 2, 3]                       # ties -> lower ids
        ok &= 0 not in ids[5] and 1 not in ids[5]                # -inf never chosen first
        ok &= 4 not in ids[6]                                    # NaN ranks last
        ok &= np.all(w[7] == 0.0)                                # no mass
        ok &= bool(np.all(np.abs(w[:7].sum(axis=1) - 1.0) < 1e-12))
        ok &= ids[8, 0] == 5
    ids4, w4 = oracle.route(l[4:5], 4, oracle.ROUTE_SOFTMAX)
    ok &= np.allclose(w4, 0.25, rtol=0, atol=1e-15)
    return _ok(ok, "router tie / -inf / NaN / no-mass rows")


def pin_route_shift_invariance():
    l = router_logits()[:3]
    ids, w = oracle.route(l, 5, oracle.ROUTE_SOFTMAX)
    ids2, w2 = oracle.route(l + np.float32(8.0), 5, oracle.ROUTE_SOFTMAX)
    idsg, _ = oracle.route(l, 5, oracle.ROUTE_SIGMOID)
    ok = np.array_equal(ids, ids2) and np.allclose(w, w2, rtol=1e-5) and np.array_equal(ids, idsg)
    return _ok(ok, "softmax weights not shift invariant or kinds choose differently")


def pin_route_vs_generator():
    """The generator's routing (its own FP64 top-k over the same draws) must
    agree with the oracle's router on the FP32-rounded logits."""
    ok = True
    for (T, E, k, kind, masked, okind) in ((64, 8, 2, gen.ROUTE_SOFTMAX, 0, oracle.ROUTE_SOFTMAX),
                                          (256, 256, 8, gen.ROUTE_SIGMOID_NORMAL, 0, oracle.ROUTE_SIGMOID),
                                          (512, 256, 8, gen.ROUTE_ZIPF, 8, oracle.ROUTE_SIGMOID)):
        ids_g, w_g = gen.make_routing(T, E, k, kind, 0, masked)
        ids_o, w_o = oracle.route(gen.make_logits(T, E, kind, 0, masked), k, okind)
        ok &= np.array_equal(ids_g, ids_o)
        ok &= np.allclose(w_g, w_o, rtol=1e-5, atol=1e-7)
    return _ok(ok, "oracle router disagrees with the generator's routing")


# ----------------------------------------------------------------- layer ---

SMALL_CASES = [
    # (E, k, H, I, T, route, rho, outlier_frac)
    (8, 2, 256, 128, 64, gen.ROUTE_SOFTMAX, 1.0, 0.0),
    (4, 3, 384, 192, 24, gen.ROUTE_SIGMOID_NORMAL, 2.5, 0.1),
    (3, 1, 256, 64, 16, gen.ROUTE_SIGMOID_NORMAL, 1.0, 0.1),
    (6, 6, 256, 256, 8, gen.ROUTE_SIGMOID_UNIFORM, 2.5, 0.2),
    # top-8, as in the GLM-class layer
    (10, 8, 256, 128, 12, gen.ROUTE_SIGMOID_NORMAL, 2.5, 0.1),
    # the tensor-sliced share's shape (H=5120, I=192 padded to 256), few experts
    (3, 2, 5120, 192, 6, gen.ROUTE_SIGMOID_NORMAL, 1.0, 0.2),
    (12, 8, 5120, 192, 4, gen.ROUTE_SIGMOID_NORMAL, 1.0, 0.25),
]


def small_case(case, seed=0):
    E, k, H, I, T, route, rho, of = case
    layer = gen.make_layer(E, H, I, seed=seed)
    x, _ = gen.make_tokens(T, H, seed=seed, outlier_frac=of)
    ids, w = gen.make_routing(T, E, k, route, seed=seed)
    return layer, x, ids, w, rho


def rel_l2_rows(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    num = np.linalg.norm(a - b, axis=1)
    den = np.linalg.norm(b, axis=1)
    return np.where(den > 0, num / np.where(den > 0, den, 1), num)


def pin_ffn_vs_bruteforce(tol=2e-3):
    worst = 0.0
    for case in SMALL_CASES:
        layer, x, ids, w, rho = small_case(case)
        out = oracle.forward(layer, x, ids, w, rho, oracle.OUT_F32)
        ref = oracle.bruteforce_fp64(layer, x, ids, w, rho, True)
        if not np.all(np.isfinite(out)):
            return _ok(False, f"non-finite output in case {case}")
        worst = max(worst, float(rel_l2_rows(out, ref).max()))
    return _ok(worst <= tol, f"worst per-row rel L2 {worst:.3g}")


def pin_down_combine_reproduces_forward():
    """The continuation used by the staged GPU comparisons: down_combine fed
    with forward's own h codes and scales gives forward's y and output rows
    bit for bit (routed layers in both output types, and with a shared slot)."""
    ok, detail = True, ""
    cases = [(small_case(c), 0) for c in SMALL_CASES]
    layer, x, _, _, ids_x, w_x, _ = shared_case()
    cases.append(((layer, x, ids_x, w_x, 2.5), 1))
    for (layer, x, ids, w, rho), n_shared in cases:
        for od in (oracle.OUT_F32, oracle.OUT_BF16):
            out, d = oracle.forward(layer, x, ids, w, rho, od, debug=True, n_shared=n_shared)
            out2, y2 = oracle.down_combine(layer, d["hq"], d["sh"], ids, w, rho, od, n_shared=n_shared)
            same_y = np.array_equal(y2.view(np.uint32), d["y"].view(np.uint32))
            same_o = np.array_equal(out2.view(np.uint8), out.view(np.uint8))
            if not (same_y and same_o):
                ok, detail = False, f"E={layer.E} H={layer.H} I={layer.I} od={od} y={same_y} out={same_o}"
    return _ok(ok, detail)


def _torch_qdq(v64: np.ndarray) -> np.ndarray:
    """Per-row 128-group quantise-dequantise with torch's float8 cast (FP32)."""
    t = torch.from_numpy(np.ascontiguousarray(v64, np.float32))
    g = t.view(t.shape[0], -1, 128)
    amax = g.abs().amax(dim=-1, keepdim=True)
    s = amax / 448.0
    q = (g / s.clamp_min(torch.finfo(torch.float32).tiny)).to(torch.float8_e4m3fn).float()
    q = torch.where(amax == 0, torch.zeros_like(q), q)
    return (q.double() * s.double()).view(t.shape).numpy()


def _dequant(codes, scales, rows, cols):
    """Weights: codes u8[rows][cols] times their 128x128 block scales."""
    d = torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).double().numpy()
    s = np.repeat(np.repeat(scales.astype(np.float64), 128, 0), 128, 1)[:rows, :cols]
    return d * s


def _dequant_rows(codes, scales):
    """Activations: codes u8[rows][cols] times their per-row 128-group scales."""
    d = torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).double().numpy()
    return d * np.repeat(scales.astype(np.float64), 128, 1)


def pin_dense_textbook(tol=2e-3):
    """E=1, k=1, w=1, rho=1 reduces the layer to one dense gated FFN."""
    H, I, T = 256, 192, 32
    layer = gen.make_layer(1, H, I, seed=7)
    x, _ = gen.make_tokens(T, H, seed=7, outlier_frac=0.1)
    ids = np.zeros((T, 1), np.int32)
    w = np.ones((T, 1), np.float32)
    out = oracle.forward(layer, x, ids, w, 1.0, oracle.OUT_F32)
    xf = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).double().numpy()
    xa = _torch_qdq(xf)
    G = _dequant(layer.gate[0], layer.gate_scale[0], I, H)
    U = _dequant(layer.up[0], layer.up_scale[0], I, H)
    D = _dequant(layer.down[0], layer.down_scale[0], H, I)
    g = xa @ G.T
    u = xa @ U.T
    h = g / (1 + np.exp(-g)) * u
    Ip = 256
    hp = np.zeros((T, Ip))
    hp[:, :I] = h
    ha = _torch_qdq(hp)[:, :I]
    ref = ha @ D.T
    err = float(rel_l2_rows(out, ref).max())
    return _ok(err <= tol, f"worst rel L2 {err:.3g}")


def integer_exact_case(I=192, seed=8):
    """Weights are small integers, scales powers of two, and every 128-group of
    x holds one 448 (so the activation scale is exactly 1 and the codes are the
    integers themselves): every gate/up sum is exact in FP32 in any order."""
    rng = np.random.default_rng(seed)
    E, H, T, k = 3, 256, 12, 2
    nI, nH = (I + 127) // 128, H // 128

    def int_codes(shape):
        vals = rng.integers(-8, 9, shape).astype(np.float32)
        return torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()

    gate = int_codes((E, I, H))
    up = int_codes((E, I, H))
    down = int_codes((E, H, I))
    pw = lambda shape: np.exp2(-rng.integers(2, 7, shape)).astype(np.float32)
    layer = gen.Layer(E, H, I, gate, up, down, pw((E, nI, nH)), pw((E, nI, nH)), pw((E, nH, nI)))
    xv = rng.integers(-16, 17, (T, H)).astype(np.float32)
    xv[:, ::128] = 448.0
    x = torch.from_numpy(xv).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    w = np.full((T, k), 0.5, np.float32)
    return layer, x, xv, ids, w


def pin_integer_exact_gate_up():
    ok = True
    for I in (128, 192, 256):
        layer, x, xv, ids, w = integer_exact_case(I)
        _, d = oracle.forward(layer, x, ids, w, 1.0, oracle.OUT_F32, debug=True)
        E, H = layer.E, layer.H
        Ip = 128 * ((I + 127) // 128)
        k = ids.shape[1]
        gu = d["gu"]
        perm = d["perm"]
        xi = xv.astype(np.int64)
        for p in range(perm.size):
            t, j = divmod(int(perm[p]), k)
            e = int(ids[t, j])
            ref = np.zeros(2 * Ip)
            for half, (W, S) in enumerate(((layer.gate, layer.gate_scale), (layer.up, layer.up_scale))):
                Wi = torch.from_numpy(W[e]).view(torch.float8_e4m3fn).float().numpy().astype(np.int64)
                for kb in range(H // 128):
                    part = Wi[:, kb * 128:(kb + 1) * 128] @ xi[t, kb * 128:(kb + 1) * 128]
                    sc = np.repeat(S[e][:, kb].astype(np.float64), 128)[:I]
                    ref[half * Ip: half * Ip + I] += part * sc
            if not np.array_equal(gu[p].astype(np.float64), ref):
                ok = False
    return _ok(ok, "gate/up not bit-exact on the integer case")


def pin_down_vs_matmul(tol=1e-5):
    layer, x, ids, w, rho = small_case(SMALL_CASES[1])
    _, d = oracle.forward(layer, x, ids, w, rho, oracle.OUT_F32, debug=True)
    H, I = layer.H, layer.I
    Ip = 128 * ((I + 127) // 128)
    k = ids.shape[1]
    worst = 0.0
    for e in range(layer.E):
        lo, hi = d["offsets"][e], d["offsets"][e + 1]
        if hi == lo:
            continue
        hdq = _dequant_rows(d["hq"][lo:hi], d["sh"][lo:hi])
        Dp = np.zeros((H, Ip))
        Dp[:, :I] = _dequant(layer.down[e], layer.down_scale[e], H, I)
        ref = hdq @ Dp.T
        worst = max(worst, float(rel_l2_rows(d["y"][lo:hi], ref).max()))
    return _ok(worst <= tol, f"worst rel L2 {worst:.3g}")


def pin_activation_from_gu():
    """h codes equal a torch re-quantisation of silu(g)*u from the oracle's own
    gate/up outputs, up to one code step where FP32 rounding of h differs."""
    layer, x, ids, w, rho = small_case(SMALL_CASES[1])
    _, d = oracle.forward(layer, x, ids, w, rho, oracle.OUT_F32, debug=True)
    Ip = d["hq"].shape[1]
    g = torch.from_numpy(d["gu"][:, :Ip]).double()
    u = torch.from_numpy(d["gu"][:, Ip:]).double()
    h = (torch.nn.functional.silu(g) * u).numpy()
    ref = _torch_qdq(h)
    got = _dequant_rows(d["hq"], d["sh"])
    err = float(rel_l2_rows(got, ref).max())
    return _ok(err <= 1e-2, f"worst rel L2 {err:.3g}")


def _f32_nearest(x):
    """The FP32 value nearest to the mpmath number x (ties to even)."""
    import mpmath
    if abs(x) >= mpmath.mpf(2) ** 128 - mpmath.mpf(2) ** 103:  # rounds to infinity
        return np.float32(np.inf) if x > 0 else np.float32(-np.inf)
    f = np.float32(float(x))
    best = f
    for c in (np.nextafter(f, np.float32(-np.inf)), np.nextafter(f, np.float32(np.inf))):
        dc, db = abs(mpmath.mpf(float(c)) - x), abs(mpmath.mpf(float(best)) - x)
        if dc < db or (dc == db and (int(c.view(np.uint32)) & 1) == 0):
            best = c
    return best


def pin_silu_exponential_correctly_rounded():
    """silu(g) * u = (g / (1 + e)) * u in FP32 with e the correctly rounded
    FP32 value of e^-g: checked against a 60-digit mpmath exponential rounded
    to FP32 by comparison with both neighbours, then numpy's IEEE FP32 add,
    divide and multiply."""
    import mpmath
    mpmath.mp.dps = 60
    rng = np.random.default_rng(31)
    g = np.concatenate([rng.standard_normal(1500) * 3, rng.uniform(-90, 90, 300),
                        np.float32([0.0, -0.0, 1e-30, -1e-30, 88.0, -87.0, -103.0, 20.5])]).astype(np.float32)
    u = rng.standard_normal(g.size).astype(np.float32)
    got = oracle.silu_mul(g, u)
    bad = 0
    for gi, ui, hi in zip(g, u, got):
        e = _f32_nearest(mpmath.exp(-mpmath.mpf(float(gi))))
        ref = np.float32(np.float32(gi) / np.float32(np.float32(1.0) + e)) * ui
        if ref.view(np.uint32) != np.float32(hi).view(np.uint32) and not (np.isnan(ref) and np.isnan(hi)):
            bad += 1
    return _ok(bad == 0, f"{bad} of {g.size} values differ")


def pin_a16_vs_bruteforce(tol=4e-3):
    """The W8A16 form against the dense FP64 evaluation without activation
    quantisation.  tol = 2 x 2^-9: the BF16 rounding of h (relative error at
    most 2^-9 per element, which the FP64 evaluation does not apply), doubled
    for the FP32 sums; W8A8 is ~5e-2 away on the same cases."""
    worst = 0.0
    for case in SMALL_CASES:
        layer, x, ids, w, rho = small_case(case)
        out = oracle.forward_a16(layer, x, ids, w, rho, oracle.OUT_F32)
        ref = oracle.bruteforce_fp64(layer, x, ids, w, rho, False)
        if not np.all(np.isfinite(out)):
            return _ok(False, f"non-finite output in case {case}")
        worst = max(worst, float(rel_l2_rows(out, ref).max()))
    return _ok(worst <= tol, f"worst per-row rel L2 {worst:.3g}")


def pin_a16_activation_from_gu():
    """W8A16 h (BF16 bits) equals torch's BF16 rounding of silu(g)*u computed
    in FP64 from the oracle's own gate/up, except where the FP32 h of the
    oracle sits within an FP32 ulp of a BF16 tie (one BF16 step) and where
    e^-g overflows FP32 (g < -88.7: the FP32 SiLU is 0, the FP64 one below
    1e-36)."""
    layer, x, ids, w, rho = small_case(SMALL_CASES[1])
    _, d = oracle.forward_a16(layer, x, ids, w, rho, oracle.OUT_F32, debug=True)
    Ip = d["hb"].shape[1]
    g = torch.from_numpy(d["gu"][:, :Ip]).double()
    u = torch.from_numpy(d["gu"][:, Ip:]).double()
    ref_t = (torch.nn.functional.silu(g) * u).to(torch.bfloat16)
    ref = ref_t.view(torch.int16).numpy().view(np.uint16)
    got = d["hb"]
    tiny = (np.abs(oracle.bf16_to_f32(got)) < 1e-30) & (np.abs(ref_t.float().numpy()) < 1e-30)
    diff = (got != ref) & ~tiny
    steps = np.abs(got.astype(np.int64) - ref.astype(np.int64))[diff]
    frac = float(diff.mean())
    return _ok(frac <= 1e-3 and (steps.size == 0 or steps.max() == 1),
               f"{int(diff.sum())} of {diff.size} BF16 values differ")


def pin_a16_exact_inputs_match_a8():
    """When every 128-group of x is already E4M3 at scale 1 (values from the
    decoded codes, one of +-448 in each group), the W8A8 quantisation of x is
    lossless, so the W8A16 gate/up equal the W8A8 ones bit for bit."""
    layer, _, ids, w, rho = small_case(SMALL_CASES[1])
    T, H = ids.shape[0], layer.H
    rng = np.random.default_rng(21)
    codes = rng.integers(0, 0x7F, size=(T, H)).astype(np.uint8) | (rng.integers(0, 2, size=(T, H)).astype(np.uint8) << 7)
    xv = oracle.e4m3_decode(codes).astype(np.float32)
    xv[:, ::128] = np.where(rng.integers(0, 2, size=(T, H // 128)) == 1, 448.0, -448.0)
    xb = oracle.f32_to_bf16(xv)
    _, d8 = oracle.forward(layer, xb, ids, w, rho, oracle.OUT_F32, debug=True)
    _, d16 = oracle.forward_a16(layer, xb, ids, w, rho, oracle.OUT_F32, debug=True)
    ok = np.array_equal(d8["gu"], d16["gu"]) and np.all(d8["sx"] == 1.0)
    return _ok(ok, "W8A16 gate/up differ from W8A8 on lossless inputs")


def pin_linearity():
    layer, x, ids, w, _ = small_case(SMALL_CASES[1])
    o1 = oracle.forward(layer, x, ids, w, 1.0, oracle.OUT_F32)
    o2 = oracle.forward(layer, x, ids, w, 2.0, oracle.OUT_F32)
    ow = oracle.forward(layer, x, ids, (w * 2).astype(np.float32), 1.0, oracle.OUT_F32)
    ok = np.array_equal(o2, o1 * 2) and np.array_equal(ow, o1 * 2)
    return _ok(ok, "not linear in rho / w")


def pin_permutation_equivariance():
    layer, x, ids, w, rho = small_case(SMALL_CASES[0])
    rng = np.random.default_rng(9)
    pi = rng.permutation(x.shape[0])
    o = oracle.forward(layer, x, ids, w, rho, oracle.OUT_BF16)
    op = oracle.forward(layer, x[pi], ids[pi], w[pi], rho, oracle.OUT_BF16)
    return _ok(np.array_equal(o[pi], op), "permuting tokens does not permute rows")


def pin_rows_independent():
    layer, x, ids, w, rho = small_case(SMALL_CASES[1])
    o = oracle.forward(layer, x, ids, w, rho, oracle.OUT_F32)
    parts = [oracle.forward(layer, x[a:b], ids[a:b], w[a:b], rho, oracle.OUT_F32)
             for a, b in ((0, 1), (1, 10), (10, x.shape[0]))]
    return _ok(np.array_equal(o, np.concatenate(parts)), "rows depend on the call")


def pin_skip_slot_equals_removed():
    layer, x, ids, w, rho = small_case(SMALL_CASES[1])
    ids2 = ids.copy()
    ids2[:, -1] = -1
    o_skip = oracle.forward(layer, x, ids2, w, rho, oracle.OUT_F32)
    o_less = oracle.forward(layer, x, np.ascontiguousarray(ids[:, :-1]),
                            np.ascontiguousarray(w[:, :-1]), rho, oracle.OUT_F32)
    return _ok(np.array_equal(o_skip, o_less), "skip slot is not a removed slot")


def pin_nan_row_isolation():
    layer, x, ids, w, rho = small_case(SMALL_CASES[1])
    o = oracle.forward(layer, x, ids, w, rho, oracle.OUT_F32)
    x2 = x.copy()
    x2[5, 17] = 0x7FC0      # bf16 NaN
    x2[9, 3] = 0x7F80       # bf16 +Inf
    o2 = oracle.forward(layer, x2, ids, w, rho, oracle.OUT_F32)
    others = np.ones(x.shape[0], bool)
    others[[5, 9]] = False
    ok = (np.isnan(o2[5]).all() and np.isnan(o2[9]).all()
          and np.array_equal(o2[others], o[others]))
    return _ok(ok, "NaN/Inf did not stay in its row")


def shared_case(seed=12):
    """E=4 routed experts + 1 shared (index 4), k=2 routed slots + the shared slot."""
    E, k, H, I, T = 4, 2, 256, 192, 20
    layer = gen.make_layer(E + 1, H, I, seed=seed)
    x, _ = gen.make_tokens(T, H, seed=seed, outlier_frac=0.1)
    ids, w = gen.make_routing(T, E, k, gen.ROUTE_SIGMOID_NORMAL, seed=seed)
    ids[3, 1] = -1
    ids_x = np.concatenate([ids, np.full((T, 1), E, np.int32)], axis=1)
    w_x = np.concatenate([w, np.ones((T, 1), np.float32)], axis=1)
    return layer, x, ids, w, ids_x, w_x, E


def pin_shared_vs_bruteforce(tol=2e-3):
    layer, x, ids, w, ids_x, w_x, E = shared_case()
    got = oracle.forward(layer, x, ids_x, w_x, 2.5, oracle.OUT_F32, n_shared=1)
    ref = oracle.bruteforce_fp64(layer, x, ids_x, w_x, 2.5, n_shared=1)
    worst = float(rel_l2_rows(got.astype(np.float64), ref).max())
    return _ok(worst <= tol, f"shared slot vs brute force: worst rel L2 {worst:.2e}")


def pin_shared_composition():
    """Routed output (FP32) plus the shared expert's own output, added once:
    the same bits as the layer with the shared slot."""
    layer, x, ids, w, ids_x, w_x, E = shared_case()
    got = oracle.forward(layer, x, ids_x, w_x, 2.5, oracle.OUT_F32, n_shared=1)
    routed = oracle.forward(layer, x, ids, w, 2.5, oracle.OUT_F32)
    one = gen.Layer(1, layer.H, layer.I, *(a[E:E + 1] for a in (layer.gate, layer.up, layer.down,
                                                            layer.gate_scale, layer.up_scale,
                                                            layer.down_scale)))
    T = x.shape[0]
    ys = oracle.forward(one, x, np.zeros((T, 1), np.int32), np.ones((T, 1), np.float32), 1.0,
                           oracle.OUT_F32)
    return _ok(np.array_equal((routed + ys).view(np.uint32), got.view(np.uint32)),
               "shared slot is not the routed layer plus the shared expert")


CLAMP = 0.5  # low enough that the test rows' gate / up values cross it


def pin_clamp_vs_bruteforce(tol=2e-3):
    layer, x, ids, w, rho = small_case(SMALL_CASES[1])
    oracle.set_activation_limit(CLAMP)
    try:
        got = oracle.forward(layer, x, ids, w, rho, oracle.OUT_F32)
        ref = oracle.bruteforce_fp64(layer, x, ids, w, rho)
    finally:
        oracle.set_activation_limit(0.0)
    unclamped = oracle.forward(layer, x, ids, w, rho, oracle.OUT_F32)
    worst = float(rel_l2_rows(got.astype(np.float64), ref).max())
    active = float(rel_l2_rows(got.astype(np.float64), unclamped.astype(np.float64)).max())
    return _ok(worst <= tol and active > 1e-2,
               f"clamped vs brute force {worst:.2e}; clamp changes rows by {active:.2e}")


def pin_clamp_activation_from_gu():
    layer, x, ids, w, rho = small_case(SMALL_CASES[1])
    oracle.set_activation_limit(CLAMP)
    try:
        _, d = oracle.forward(layer, x, ids, w, rho, oracle.OUT_F32, debug=True)
    finally:
        oracle.set_activation_limit(0.0)
    Ip = d["gu"].shape[1] // 2
    g = np.minimum(d["gu"][:, :Ip].astype(np.float64), CLAMP)
    u = np.clip(d["gu"][:, Ip:].astype(np.float64), -CLAMP, CLAMP)
    h = g / (1.0 + np.exp(-g)) * u
    q, s = oracle.quantize_rows(h.astype(np.float32))
    dec = oracle.e4m3_decode(np.arange(256, dtype=np.uint8)).astype(np.float64)
    back = dec[d["hq"]] * np.repeat(d["sh"].astype(np.float64), 128, axis=1)
    rel = np.abs(back - h).max() / np.abs(h).max()
    same = (q != d["hq"]).mean()
    return _ok(rel < 0.07 and same < 1e-3, f"clamped h: max rel {rel:.3f}, code mismatch {same:.2e}")


def pin_clamp_large_limit_is_unclamped():
    layer, x, ids, w, rho = small_case(SMALL_CASES[1])
    base = oracle.forward(layer, x, ids, w, rho, oracle.OUT_F32)
    oracle.set_activation_limit(1e30)
    try:
        big = oracle.forward(layer, x, ids, w, rho, oracle.OUT_F32)
    finally:
        oracle.set_activation_limit(0.0)
    return _ok(np.array_equal(base.view(np.uint32), big.view(np.uint32)), "a huge limit changed bits")


def slice_case(seed=21):
    return gen.make_layer(3, 256, 384, seed=seed)


def pin_slice_aligned_is_plain():
    l = slice_case()
    ok = True
    for off, n in ((0, 192), (128, 192), (256, 128), (128, 256)):
        a = oracle.slice_layer(l, off, n)
        nb = (n + 127) // 128
        ok &= np.array_equal(a.gate, l.gate[:, off:off + n]) and np.array_equal(a.up, l.up[:, off:off + n])
        ok &= np.array_equal(a.down, l.down[:, :, off:off + n])
        ok &= np.array_equal(a.gate_scale, l.gate_scale[:, off // 128:off // 128 + nb])
        ok &= np.array_equal(a.down_scale, l.down_scale[:, :, off // 128:off // 128 + nb])
    return _ok(ok, "aligned slices differ from plain slicing")


def _torch_requant(v):
    """Block-requantise FP32 values [R][C] per 128x128 block with torch."""
    R, C = v.shape
    codes = np.zeros((R, C), np.uint8)
    scales = np.zeros(((R + 127) // 128, (C + 127) // 128), np.float32)
    for bi in range(scales.shape[0]):
        for bj in range(scales.shape[1]):
            blk = torch.from_numpy(np.ascontiguousarray(v[bi * 128:(bi + 1) * 128, bj * 128:(bj + 1) * 128]))
            amax = blk.abs().max()
            sc = amax / 448.0
            scales[bi, bj] = sc.item()
            if amax.item() != 0.0:
                codes[bi * 128:(bi + 1) * 128, bj * 128:(bj + 1) * 128] = \
                    (blk / sc).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, scales


def pin_slice_requant_vs_torch():
    l = slice_case()
    dec = oracle.e4m3_decode(np.arange(256, dtype=np.uint8))
    ok, worst = True, 0.0
    for off, n in ((192, 192), (64, 256), (200, 100)):
        a = oracle.slice_layer(l, off, n)
        for e in range(l.gate.shape[0]):
            for name, axis in (("gate", 0), ("up", 0), ("down", 1)):
                full = getattr(l, name)[e]
                sc = np.repeat(np.repeat(getattr(l, name + "_scale")[e], 128, 0), 128, 1)[:full.shape[0], :full.shape[1]]
                v = (dec[full] * sc).astype(np.float32)     # FP32 products, as the oracle forms them
                v = v[off:off + n] if axis == 0 else v[:, off:off + n]
                c_ref, s_ref = _torch_requant(v)
                got_c, got_s = getattr(a, name)[e], getattr(a, name + "_scale")[e]
                ok &= np.array_equal(got_c, c_ref) and np.array_equal(got_s.view(np.uint32), s_ref.view(np.uint32))
                back = dec[got_c].astype(np.float64) * np.repeat(np.repeat(got_s, 128, 0), 128, 1)[:v.shape[0], :v.shape[1]]
                worst = max(worst, float((np.abs(back - v) / np.maximum(np.abs(v), 1e-30))[np.abs(v) > 1e-4].max()))
    return _ok(ok and worst <= 1 / 16 + 1e-6, f"requant bits equal={ok}, worst rel error {worst:.4f}")


def pin_slices_add_up():
    """Two tensor-parallel shares (one aligned, one requantised) through the
    FP64 brute force add up to the full layer's output."""
    l = slice_case()
    T = 12
    x, _ = gen.make_tokens(T, l.H, seed=4)
    ids, w = gen.make_routing(T, 3, 2, gen.ROUTE_SIGMOID_NORMAL, seed=4)
    full = oracle.bruteforce_fp64(l, x, ids, w, 1.0, quantize_activations=False)
    parts = sum(oracle.bruteforce_fp64(oracle.slice_layer(l, off, 192), x, ids, w, 1.0,
                                       quantize_activations=False) for off in (0, 192))
    worst = float(rel_l2_rows(parts, full).max())
    return _ok(worst <= 3e-2, f"slices add up to the full layer within {worst:.3e}")


ALL_PINS = {
    "decode_golden": pin_decode_golden,
    "decode_vs_torch": pin_decode_vs_torch,
    "decode_structure": pin_decode_structure,
    "encode_vs_torch": pin_encode_vs_torch,
    "encode_specials": pin_encode_specials,
    "encode_roundtrip": pin_encode_roundtrip,
    "encode_vs_nearest_search": pin_encode_vs_nearest_search,
    "bf16_widen_vs_torch": pin_bf16_widen_vs_torch,
    "bf16_narrow_vs_torch": pin_bf16_narrow_vs_torch,
    "quantize_vs_torch": pin_quantize_vs_torch,
    "quantize_invariants": pin_quantize_invariants,
    "plan_vs_numpy": pin_plan_vs_numpy,
    "route_ids_vs_sort": pin_route_ids_vs_sort,
    "route_weights_vs_scipy": pin_route_weights_vs_scipy,
    "route_special_rows": pin_route_special_rows,
    "route_shift_invariance": pin_route_shift_invariance,
    "route_vs_generator": pin_route_vs_generator,
    "ffn_vs_bruteforce": pin_ffn_vs_bruteforce,
    "dense_textbook": pin_dense_textbook,
    "integer_exact_gate_up": pin_integer_exact_gate_up,
    "down_vs_matmul": pin_down_vs_matmul,
    "down_combine_reproduces_forward": pin_down_combine_reproduces_forward,
    "silu_exponential_correctly_rounded": pin_silu_exponential_correctly_rounded,
    "activation_from_gu": pin_activation_from_gu,
    "linearity": pin_linearity,
    "permutation_equivariance": pin_permutation_equivariance,
    "rows_independent": pin_rows_independent,
    "skip_slot_equals_removed": pin_skip_slot_equals_removed,
    "nan_row_isolation": pin_nan_row_isolation,
    "shared_vs_bruteforce": pin_shared_vs_bruteforce,
    "shared_composition": pin_shared_composition,
    "clamp_vs_bruteforce": pin_clamp_vs_bruteforce,
    "clamp_activation_from_gu": pin_clamp_activation_from_gu,
    "clamp_large_limit_is_unclamped": pin_clamp_large_limit_is_unclamped,
    "slice_aligned_is_plain": pin_slice_aligned_is_plain,
    "slice_requant_vs_torch": pin_slice_requant_vs_torch,
    "slices_add_up": pin_slices_add_up,
    "a16_vs_bruteforce": pin_a16_vs_bruteforce,
    "a16_activation_from_gu": pin_a16_activation_from_gu,
    "a16_exact_inputs_match_a8": pin_a16_exact_inputs_match_a8,
}
