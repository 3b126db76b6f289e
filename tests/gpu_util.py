"""Helpers shared by the GPU tests: device transfer, runs through the C ABI,
per-row comparison against the oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

import fp8_blockwise_routed_amd as pkg

TOL = 2e-2  # per-row relative L2 bound on the output


def note(msg: str) -> None:
    """Name the case before a GPU step (flushed, so it survives a lost box)."""
    print(msg, flush=True)
    sys.stdout.flush()


def dev_bf16(x_bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).view(torch.bfloat16).cuda()


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def out_to_np(out: torch.Tensor) -> np.ndarray:
    if out.dtype == torch.bfloat16:
        return out.view(torch.int16).cpu().numpy().view(np.uint16)
    return out.cpu().numpy()


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def as_f64(out: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f64(out) if out.dtype == np.uint16 else out.astype(np.float64)


def run(moe: pkg.MoeFp8Prefill, x_bits, ids, w) -> np.ndarray:
    """One call through the C ABI; returns the output rows on the host (bf16
    bits as uint16, or float32)."""
    out = moe.run(dev_bf16(x_bits), dev(ids), dev(w))
    torch.cuda.synchronize()
    return out_to_np(out)


def rel_l2_rows(got, ref) -> np.ndarray:
    g = as_f64(got)
    r = as_f64(ref)
    num = np.linalg.norm(g - r, axis=1)
    den = np.linalg.norm(r, axis=1)
    return np.where(den > 0, num / np.where(den > 0, den, 1.0), num)


def assert_rows_close(got, ref, tol=TOL, what=""):
    g = as_f64(got)
    r = as_f64(ref)
    nan_g, nan_r = np.isnan(g), np.isnan(r)
    assert np.array_equal(nan_g, nan_r), f"{what}: NaN positions differ"
    finite_rows = ~nan_r.any(axis=1)
    rel = rel_l2_rows(g[finite_rows], r[finite_rows])
    zero_ref = np.linalg.norm(r[finite_rows], axis=1) == 0
    assert np.all(g[finite_rows][zero_ref] == 0), f"{what}: rows that must be zero are not"
    worst = float(rel.max()) if rel.size else 0.0
    note(f"  {what}: rows={g.shape[0]} worst rel L2 {worst:.3e} mean {float(rel.mean()) if rel.size else 0:.3e}")
    assert worst <= tol, f"{what}: worst per-row rel L2 {worst} > {tol}"
    return worst


# ---- stage-wise comparison ---------------------------------------------------
#
# The gfx950 FP8 MFMA sums a 128-wide block dot keeping about 13 bits below
# its largest product (the rest truncated), so gate/up differ from the
# oracle's FP32 sums by ~1e-5 relative.  Where such an FP32 value decides an
# E4M3 code of h near a rounding midpoint, the two sides can pick neighbouring
# codes.  Layers with one h group per row (Ip = 128), where one such flip
# would move a row by ~1%, have those decisions recomputed exactly by the
# library, so their codes and scales must equal the oracle's.  Elsewhere the
# decision is taken at the kernel's precision and the comparison is staged:
#   (1) gate/up (FP32, before the epilogue) vs the oracle: per-row rel L2;
#   (2) the kernel's h codes and scales are exact E4M3 roundings of the
#       kernel's own h = silu(g) * u (up to FP32 SiLU rounding at exact ties);
#   (3) the oracle continued from the kernel's h codes (down + combine) vs the
#       kernel's y and output rows.
# The plain end-to-end per-row error against the oracle is reported too.

GU_TOL = 1e-4        # per-row rel L2 of gate/up pre-activation vs the oracle
SILU_TIE = 1e-5      # relative distance to a code midpoint inside which FP32 SiLU rounding may decide
Y_TOL = 1e-4         # down output rows from identical h codes
OUT_TOL_F32 = 1e-4   # output rows from identical h codes (FP32 out)
OUT_TOL_BF16 = 8e-3  # output rows from identical h codes (BF16 out: one rounding)

_DEC = None


def _dec_table():
    global _DEC
    if _DEC is None:
        import oracle
        _DEC = oracle.e4m3_decode(np.arange(256, dtype=np.uint8)).astype(np.float64)
    return _DEC


def check_h_codes(hq_k, sh_k, gu_k, Ip, act_limit=0.0):
    """The kernel's h codes / scales are the E4M3 quantisation (per row and
    128-group, s = amax/448, round to nearest even) of its own h."""
    import oracle
    dec = _dec_table()
    g = gu_k[:, :Ip].astype(np.float64)
    u = gu_k[:, Ip:].astype(np.float64)
    if act_limit > 0:
        g = np.minimum(g, act_limit)
        u = np.clip(u, -act_limit, act_limit)
    h = g / (1.0 + np.exp(-g)) * u
    rows, groups = sh_k.shape
    amax = np.abs(h).reshape(rows, groups, 128).max(axis=2)
    s_ref = (amax / 448.0)
    ok_s = np.abs(sh_k - s_ref) <= SILU_TIE * np.abs(s_ref) + 1e-38
    assert ok_s.all(), f"{(~ok_s).sum()} h scales differ from amax/448 of the kernel's h"
    s = np.repeat(sh_k.astype(np.float64), 128, axis=1)
    v = np.where(s > 0, h / np.where(s > 0, s, 1.0), 0.0)
    nearest = oracle.e4m3_encode(v.astype(np.float32))
    differ = nearest != hq_k
    if differ.any():
        vd = v[differ]
        mid = 0.5 * (dec[hq_k[differ]] + dec[nearest[differ]])
        near_tie = np.abs(vd - mid) <= SILU_TIE * np.maximum(np.abs(vd), 2.0 ** -9)
        assert near_tie.all(), f"{(~near_tie).sum()} h codes are not roundings of the kernel's h"
    return int(differ.sum())


def with_shared_slot(ids, w, E_routed):
    """ids / w with the shared expert's slot (id E_routed, weight 1) appended."""
    T = ids.shape[0]
    return (np.concatenate([ids, np.full((T, 1), E_routed, np.int32)], axis=1),
            np.concatenate([w, np.ones((T, 1), np.float32)], axis=1))


def compare_with_oracle(moe, layer, x, ids, w, rho, got, what="", n_shared=0, act_limit=0.0):
    """Staged comparison of a finished run whose last pass was the whole call.
    With n_shared, ids / w already carry the shared slot column."""
    import oracle
    od = oracle.OUT_F32 if got.dtype == np.float32 else oracle.OUT_BF16
    oracle.set_activation_limit(act_limit)
    try:
        ref, d = oracle.forward(layer, x, ids, w, rho, od, debug=True, n_shared=n_shared)
    finally:
        oracle.set_activation_limit(0.0)
    Ip = 128 * ((layer.I + 127) // 128)
    n = d["hq"].shape[0]
    gu = pkg.moe_fp8_prefill_debug_gate_up(moe.handle, n, Ip)
    hq, sh, y = pkg.moe_fp8_prefill_debug_intermediates(moe.handle, n, layer.H, Ip)
    fin = np.isfinite(d["gu"]).all(axis=1)
    rel_gu = rel_l2_rows(gu[fin], d["gu"][fin])
    flips = int((hq[fin] != d["hq"][fin]).sum())
    if Ip == 128:
        # one h group per row: the library's exact-tie quantiser decides every
        # code and scale as the definition does
        ties = 0
        if flips:
            r, c = np.nonzero((hq != d["hq"]) & fin[:, None])
            note(f"  {what}: h codes differ at (row, col) {list(zip(r[:4].tolist(), c[:4].tolist()))}: "
                 f"kernel {hq[r[:4], c[:4]].tolist()} oracle {d['hq'][r[:4], c[:4]].tolist()} "
                 f"gate {d['gu'][r[:4], c[:4]].tolist()} up {d['gu'][r[:4], Ip + c[:4]].tolist()} "
                 f"kernel gate {gu[r[:4], c[:4]].tolist()} up {gu[r[:4], Ip + c[:4]].tolist()} "
                 f"scale {sh[r[:4], 0].tolist()} vs {d['sh'][r[:4], 0].tolist()}")
        assert flips == 0, f"{what}: {flips} h codes differ from the oracle's"
        assert np.array_equal(sh[fin].view(np.uint32), d["sh"][fin].view(np.uint32)), \
            f"{what}: h scales differ from the oracle's"
    else:
        ties = check_h_codes(hq[fin], sh[fin], gu[fin], Ip, act_limit)
    out2, y2 = oracle.down_combine(layer, hq, sh, ids, w, rho, od, n_shared=n_shared)
    rel_y = rel_l2_rows(y[fin], y2[fin])
    note(f"  {what}: gate/up rel L2 max {rel_gu.max() if rel_gu.size else 0:.2e}; h codes vs oracle's "
         f"{flips}/{hq[fin].size} differ ({ties} at SiLU ties); y rel max {rel_y.max() if rel_y.size else 0:.2e}")
    assert rel_gu.size == 0 or rel_gu.max() <= GU_TOL, f"{what}: gate/up off by {rel_gu.max()}"
    assert rel_y.size == 0 or rel_y.max() <= Y_TOL, f"{what}: y off by {rel_y.max()}"
    assert_rows_close(got, out2, tol=OUT_TOL_F32 if od == oracle.OUT_F32 else OUT_TOL_BF16,
                      what=f"{what} vs oracle continued from kernel h")
    rows = np.isfinite(as_f64(ref)).all(1)
    worst_plain = float(rel_l2_rows(got[rows], ref[rows]).max()) if rows.any() else 0.0
    note(f"  {what}: plain end-to-end worst per-row rel L2 {worst_plain:.3e}")
    assert worst_plain <= TOL, f"{what}: plain end-to-end worst per-row rel L2 {worst_plain} > {TOL}"
    return ref, d, worst_plain
