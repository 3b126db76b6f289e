"""GPU path vs the oracle on layers the oracle evaluates in full (GPU).

Covers: weight layout round trip (byte exact, NaN codes sanitised, I edge
padding), the plan (bit exact), the activation quantiser (bit exact), and the
end-to-end output (per-row relative L2 <= 2e-2) in BF16 and FP32 output,
across several tiles, ragged tails and the small- and multi-subtile GEMMs.
"""
import numpy as np
import pytest
import torch

import fp8_blockwise_routed_amd as pkg
import gen
import oracle
from gpu_util import TOL, assert_rows_close, compare_with_oracle, dev, dev_bf16, note, run

pytestmark = pytest.mark.gpu

# (E, k, H, I, T, route, rho, outlier_frac): small enough for the oracle in
# seconds; experts get from 0 to a few hundred rows (both GEMM variants:
# 16-row streaming and 256-row tiles, one or both halves used, ragged last
# tiles); I=192 exercises the
# zero padding to 256.
CASES = [
    ("tiny", (8, 2, 256, 128, 64, gen.ROUTE_SOFTMAX, 1.0, 0.0)),
    ("pad192", (6, 3, 512, 192, 50, gen.ROUTE_SIGMOID_NORMAL, 2.5, 0.05)),
    ("i64", (5, 2, 384, 64, 37, gen.ROUTE_SIGMOID_NORMAL, 1.0, 0.0)),
    ("many_rows", (4, 2, 256, 256, 600, gen.ROUTE_SIGMOID_UNIFORM, 2.5, 0.01)),
    ("slice_t64", (160, 8, 5120, 192, 64, gen.ROUTE_SIGMOID_NORMAL, 1.0, 0.01)),
    # ~470 rows per expert: 256-row tiles with both halves full; odd K-block
    # counts (H/128 = 3, Ip/128 = 3) and an odd count of down column blocks
    ("wide_odd", (3, 2, 384, 320, 700, gen.ROUTE_SIGMOID_UNIFORM, 2.5, 0.01)),
    # the largest K loops the library takes (H / 128 = 128 for gate_up,
    # Ip / 128 = 128 for down), 150 rows per expert (256-row tiles)
    ("max_h", (2, 2, 16384, 256, 150, gen.ROUTE_SIGMOID_NORMAL, 1.0, 0.01)),
    ("max_i", (2, 2, 256, 16384, 150, gen.ROUTE_SIGMOID_NORMAL, 1.0, 0.01)),
]


def make_case(spec, seed=0):
    E, k, H, I, T, route, rho, of = spec
    layer = gen.make_layer(E, H, I, seed=seed)
    x, _ = gen.make_tokens(T, H, seed=seed, outlier_frac=of)
    ids, w = gen.make_routing(T, E, k, route, seed=seed)
    return layer, x, ids, w, rho


@pytest.mark.parametrize("name,spec", CASES[:3])
def test_layout_round_trip(name, spec):
    layer, *_ = make_case(spec)
    # plant NaN codes: the library stores them as signed zeros
    layer.gate[0, 0, 0] = 0x7F
    layer.up[-1, -1, -1] = 0xFF
    layer.down[0, 5, 3] = 0xFF
    note(f"layout round trip {name}")
    moe = pkg.MoeFp8Prefill(layer, spec[1])
    try:
        for e in range(layer.E):
            got = pkg.moe_fp8_prefill_debug_unpack(moe.handle, e, layer.H, layer.I)
            for key in ("gate", "up", "down"):
                src = getattr(layer, key)[e].copy()
                src[src == 0x7F] = 0x00
                src[src == 0xFF] = 0x80
                assert np.array_equal(got[key], src), (e, key)
            for key in ("gate_scale", "up_scale", "down_scale"):
                assert np.array_equal(got[key].view(np.uint32), getattr(layer, key)[e].view(np.uint32))
    finally:
        moe.close()


@pytest.mark.parametrize("name,spec", CASES)
@pytest.mark.parametrize("out_dtype", [pkg.MOE_DTYPE_BF16, pkg.MOE_DTYPE_F32])
def test_end_to_end_matches_oracle(name, spec, out_dtype):
    layer, x, ids, w, rho = make_case(spec)
    k = spec[1]
    note(f"end-to-end {name} out_dtype={out_dtype} T={x.shape[0]}")
    moe = pkg.MoeFp8Prefill(layer, k, routed_scale=rho, out_dtype=out_dtype)
    try:
        got = run(moe, x, ids, w)
        assert moe.status() == pkg.MOE_OK
        T = x.shape[0]
        counts, offsets, perm, inv = pkg.moe_fp8_prefill_debug_plan(moe.handle, layer.E, T * k)
        xq, sx = pkg.moe_fp8_prefill_debug_activations(moe.handle, T, layer.H)
    finally:
        moe.close()
    ref, d = oracle.forward(layer, x, ids, w, rho,
                            oracle.OUT_F32 if out_dtype == pkg.MOE_DTYPE_F32 else oracle.OUT_BF16,
                            debug=True)
    # integer work: bit exact
    assert np.array_equal(counts, d["counts"])
    assert np.array_equal(offsets, d["offsets"])
    assert np.array_equal(perm, d["perm"])
    assert np.array_equal(inv, d["inv"])
    # the activation quantiser decides codes in FP32 with IEEE division on both sides
    assert np.array_equal(xq, d["xq"])
    assert np.array_equal(sx.view(np.uint32), d["sx"].view(np.uint32))
    # plain end-to-end bound, every layer
    assert_rows_close(got, ref, tol=TOL, what=f"{name}/{out_dtype}")


@pytest.mark.parametrize("name,spec", CASES)
def test_stages_match_oracle(name, spec):
    """gate/up within GU_TOL, every h code a valid rounding, and the rest of
    the layer from the kernel's h codes within FP32 / BF16 rounding."""
    layer, x, ids, w, rho = make_case(spec)
    for od in (pkg.MOE_DTYPE_F32, pkg.MOE_DTYPE_BF16):
        note(f"stages {name} out_dtype={od}")
        moe = pkg.MoeFp8Prefill(layer, spec[1], routed_scale=rho, out_dtype=od)
        try:
            got = run(moe, x, ids, w)
            compare_with_oracle(moe, layer, x, ids, w, rho, got, what=f"{name}/{od}")
        finally:
            moe.close()


def test_skip_slots_and_bad_ids():
    layer, x, ids, w, rho = make_case(CASES[1][1])
    k = CASES[1][1][1]
    ids = ids.copy()
    ids[3, 1] = -1          # skip slot
    ids[7, :] = -5          # a token with no routed slot: output row is zero
    ids[11, 2] = layer.E    # bad id: skipped and reported
    note("skip slots and bad ids")
    moe = pkg.MoeFp8Prefill(layer, k, routed_scale=rho, out_dtype=pkg.MOE_DTYPE_F32)
    try:
        got = run(moe, x, ids, w)
        assert moe.status() == pkg.MOE_ERR_BAD_EXPERT_ID
        assert moe.status() == pkg.MOE_OK          # cleared by the first read
        counts, offsets, perm, inv = pkg.moe_fp8_prefill_debug_plan(moe.handle, layer.E, x.shape[0] * k)
    finally:
        moe.close()
    ref, d = oracle.forward(layer, x, ids, w, rho, oracle.OUT_F32, debug=True)
    assert d["n_bad"] == 1
    assert np.array_equal(perm, d["perm"]) and np.array_equal(inv, d["inv"])
    assert np.all(got[7] == 0)
    assert_rows_close(got, ref, what="skip/bad")


def test_nan_and_inf_stay_in_their_rows():
    layer, x, ids, w, rho = make_case(CASES[0][1])
    x = x.copy()
    x[5, 17] = 0x7FC0   # NaN
    x[9, 3] = 0xFF80    # -Inf
    note("nan/inf isolation")
    moe = pkg.MoeFp8Prefill(layer, CASES[0][1][1], routed_scale=rho, out_dtype=pkg.MOE_DTYPE_F32)
    try:
        got = run(moe, x, ids, w)
        clean = x.copy()
        clean[5] = 0
        clean[9] = 0
        got_clean = run(moe, clean, ids, w)
    finally:
        moe.close()
    ref = oracle.forward(layer, x, ids, w, rho, oracle.OUT_F32)
    assert np.isnan(got[5]).all() and np.isnan(got[9]).all()
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    others = np.ones(x.shape[0], bool)
    others[[5, 9]] = False
    assert np.array_equal(got[others], got_clean[others])


def test_empty_and_single_row_calls():
    layer, x, ids, w, rho = make_case(CASES[0][1])
    note("T=0 and T=1")
    moe = pkg.MoeFp8Prefill(layer, CASES[0][1][1], routed_scale=rho, out_dtype=pkg.MOE_DTYPE_F32)
    try:
        out = torch.full((1, layer.H), 7.0, device="cuda")
        rc = pkg.moe_fp8_prefill_run(moe.handle, dev_bf16(x[:1]), dev(ids[:1]), dev(w[:1]), 0, out)
        torch.cuda.synchronize()
        assert rc == pkg.MOE_OK and torch.all(out == 7.0)
        one = run(moe, x[4:5], ids[4:5], w[4:5])
        full = run(moe, x, ids, w)
    finally:
        moe.close()
    assert np.array_equal(one[0].view(np.uint32), full[4].view(np.uint32))


def test_internal_chunking_is_invisible():
    """T > max_rows runs in passes of max_rows rows; every row's bits equal
    those of the same row in a one-pass call."""
    spec = CASES[3][1]  # 600 rows, up to a few hundred rows per expert
    layer, x, ids, w, rho = make_case(spec)
    note("internal chunking max_rows=97 vs 1024")
    small = pkg.MoeFp8Prefill(layer, spec[1], routed_scale=rho, max_rows=97, out_dtype=pkg.MOE_DTYPE_F32)
    big = pkg.MoeFp8Prefill(layer, spec[1], routed_scale=rho, max_rows=1024, out_dtype=pkg.MOE_DTYPE_F32)
    try:
        a = run(small, x, ids, w)
        b = run(big, x, ids, w)
    finally:
        small.close()
        big.close()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_rows_do_not_depend_on_the_call():
    """Row alone, row among others, odd splits and a token permutation all give
    the same bits per row."""
    spec = CASES[3][1]
    layer, x, ids, w, rho = make_case(spec)
    note("row invariance small")
    moe = pkg.MoeFp8Prefill(layer, spec[1], routed_scale=rho, out_dtype=pkg.MOE_DTYPE_BF16)
    try:
        full = run(moe, x, ids, w)
        parts = np.concatenate([run(moe, x[a:b], ids[a:b], w[a:b])
                                for a, b in ((0, 1), (1, 300), (300, 599), (599, 600))])
        rng = np.random.default_rng(5)
        pi = rng.permutation(x.shape[0])
        perm_out = run(moe, x[pi], ids[pi], w[pi])
        again = run(moe, x, ids, w)
    finally:
        moe.close()
    assert np.array_equal(full, parts)
    assert np.array_equal(full[pi], perm_out)
    assert np.array_equal(full, again)


def test_output_guard_words_untouched():
    spec = CASES[0][1]
    layer, x, ids, w, rho = make_case(spec)
    T, H = x.shape
    note("guard words")
    moe = pkg.MoeFp8Prefill(layer, spec[1], routed_scale=rho, out_dtype=pkg.MOE_DTYPE_BF16)
    try:
        pad = 64  # elements (128 bytes) of guard on each side
        buf = torch.full((T * H + 2 * pad,), -12345, dtype=torch.int16, device="cuda")
        out = buf[pad:pad + T * H]
        rc = pkg.moe_fp8_prefill_run(moe.handle, dev_bf16(x), dev(ids), dev(w), T, out.data_ptr())
        torch.cuda.synchronize()
        assert rc == pkg.MOE_OK
        host = buf.cpu().numpy()
    finally:
        moe.close()
    assert np.all(host[:pad] == -12345) and np.all(host[-pad:] == -12345)


def test_stage_timing_records():
    """Per-launch timing: one row of MOE_NUM_STAGES non-negative intervals per
    pass; the 256-row group carries time when experts have more than 128
    rows (E=4, ~300 rows each) and the streaming group when none has 1-16."""
    spec = CASES[3][1]
    layer, x, ids, w, rho = make_case(spec)
    note("stage timing")
    moe = pkg.MoeFp8Prefill(layer, spec[1], routed_scale=rho, out_dtype=pkg.MOE_DTYPE_BF16)
    try:
        pkg.moe_fp8_prefill_set_timing(moe.handle, True)
        for _ in range(3):
            run(moe, x, ids, w)
        st = pkg.moe_fp8_prefill_read_timing(moe.handle)
        # only two stages: the others read -1, the two agree with the full record
        pkg.moe_fp8_prefill_set_timing_stages(moe.handle, ["gate_up_wide", "combine"])
        for _ in range(2):
            run(moe, x, ids, w)
        part = pkg.moe_fp8_prefill_read_timing(moe.handle)
        pkg.moe_fp8_prefill_set_timing(moe.handle, False)
        run(moe, x, ids, w)
        none = pkg.moe_fp8_prefill_read_timing(moe.handle)
    finally:
        moe.close()
    assert st.shape == (3, pkg.MOE_NUM_STAGES)
    assert np.all(st >= 0)
    s = dict(zip(pkg.STAGES, st.mean(axis=0)))
    assert s["gate_up_wide"] > s["gate_up_stream"] and s["down_wide"] > s["down_stream"]
    assert part.shape == (2, pkg.MOE_NUM_STAGES) and none.shape[0] == 0
    timed = [pkg.STAGES.index("gate_up_wide"), pkg.STAGES.index("combine")]
    others = [i for i in range(pkg.MOE_NUM_STAGES) if i not in timed]
    assert np.all(part[:, others] == -1) and np.all(part[:, timed] > 0)
    gu = part[:, timed[0]].mean()
    assert 0.5 * s["gate_up_wide"] < gu < 2.0 * s["gate_up_wide"]
