"""The full-size workloads on the GPU (GPU).

Layer E=256, top-8, H=6144, I=2048 (9.002 GiB of FP8 codes and FP32 scales)
at T=256 (sigmoid top-8, rho=2.5, 1% outlier rows), T=4096 (uniform routing
logits) and T=8192 (Zipf(1.2) popularity with 8 experts never chosen), run
exactly as the benchmark runs them (one handle, max_rows=8192, one call per
batch); the W8A16 decode path on the same layer at T=16; and the E=160,
H=5120, I=192 slice at T=16/64/1024.

Integer work (plan, activation codes) is compared in full, bit for bit.  The
output is compared stage by stage as in gpu_util on every row at T=256 and
on the slice, and at T=4096 and T=8192 on at least 64 rows that reach every
GEMM tile kind (streaming, 128-row, 256-row, ragged last tiles, the largest
expert) and the outlier rows; the oracle evaluates that token subset, whose
rows equal the full call's (rows are independent).  Row
invariance is checked bit for bit: 1x8192 vs 2x4096 vs 4102+4090 vs 1+8191,
a row alone vs inside a 4096-row call, a token permutation, repeated calls.
"""
import hashlib

import numpy as np
import pytest
import torch

import fp8_blockwise_routed_amd as pkg
import gen
import oracle
from gpu_util import (GU_TOL, OUT_TOL_BF16, TOL, Y_TOL, as_f64, assert_rows_close, check_h_codes,
                      dev, dev_bf16, note, out_to_np, rel_l2_rows)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def glm():
    wl = gen.GLM_T256
    note("generating the E=256 H=6144 I=2048 layer (9.0 GiB)")
    layer = gen.make_layer(wl.E, wl.H, wl.I, seed=wl.seed)
    note("creating the handle")
    moe = pkg.MoeFp8Prefill(layer, wl.k, routed_scale=wl.rho, max_rows=8192,
                            out_dtype=pkg.MOE_DTYPE_BF16)
    yield layer, moe
    moe.close()


def call(moe, x, ids, w):
    out = moe.run(dev_bf16(x), dev(ids), dev(w))
    torch.cuda.synchronize()
    return out_to_np(out)


def tile_kind_rows(ids, E, outlier, n_min=64, seed=12):
    """At least n_min token rows that together reach every GEMM tile kind of
    the call: experts with 1..16 rows (streaming), 17..128 (one 128-row
    tile) and more (256-row tiles), rows in the ragged last 256-row tile of
    an expert, rows of the largest expert (first, middle, last), and the
    outlier rows; the rest drawn at random."""
    T, k = ids.shape
    counts, offsets, perm, inv, _ = oracle.plan(ids, E)
    rng = np.random.default_rng(seed)
    pick = []

    def add(tokens, n):
        tokens = [int(t) for t in tokens if int(t) not in pick]
        pick.extend(tokens[:n])

    for lo, hi in ((1, 16), (17, 128), (129, 1 << 30)):
        experts = np.nonzero((counts >= lo) & (counts <= hi))[0]
        if experts.size:
            sel = rng.permutation(experts)[:16]
            add([perm[offsets[e]] // k for e in sel], 12)
    ragged = [e for e in np.nonzero(counts > 128)[0] if counts[e] % 256]
    for e in ragged[:12]:
        add([perm[offsets[e] + counts[e] - 1] // k], 1)
    big = int(np.argmax(counts))
    add([perm[offsets[big] + q] // k for q in (0, counts[big] // 2, counts[big] - 1)], 3)
    add(np.nonzero(outlier)[0], 4)
    rest = rng.permutation(T)
    add(rest, max(0, n_min - len(pick)))
    return np.array(sorted(pick))


def stagewise_on_sample(moe, layer, x, ids, w, rho, got, S, what):
    """Oracle on the token subset S, compared stage by stage with the rows of
    the full call that belong to those tokens."""
    k = ids.shape[1]
    T = x.shape[0]
    Ip = 128 * ((layer.I + 127) // 128)
    od = oracle.OUT_BF16 if got.dtype == np.uint16 else oracle.OUT_F32
    ref, d = oracle.forward(layer, x[S], ids[S], w[S], rho, od, debug=True)
    assert_rows_close(got[S], ref, tol=TOL, what=f"{what} plain")
    counts, offsets, perm, inv = pkg.moe_fp8_prefill_debug_plan(moe.handle, layer.E, T * k)
    n_all = int(offsets[-1])
    # map the subset's sorted positions to the full call's positions
    f_sub = d["perm"]
    t_sub, j = f_sub // k, f_sub % k
    p_full = inv[S[t_sub] * k + j]
    assert np.all(p_full >= 0)
    gu = pkg.moe_fp8_prefill_debug_gate_up(moe.handle, n_all, Ip)[p_full]
    hq, sh, _ = pkg.moe_fp8_prefill_debug_intermediates(moe.handle, n_all, layer.H, Ip)
    hq, sh = hq[p_full], sh[p_full]
    rel_gu = rel_l2_rows(gu, d["gu"])
    ties = check_h_codes(hq, sh, gu, Ip)
    flips = int((hq != d["hq"]).sum())
    out2, _ = oracle.down_combine(layer, hq, sh, ids[S], w[S], rho, od)
    note(f"  {what}: gate/up rel max {rel_gu.max():.2e}, h codes vs oracle's {flips}/{hq.size} "
         f"differ ({ties} at SiLU ties)")
    assert rel_gu.max() <= GU_TOL
    assert_rows_close(got[S], out2, tol=OUT_TOL_BF16 if od == oracle.OUT_BF16 else 1e-4,
                      what=f"{what} continued from kernel h")


def test_glm_t256(glm):
    layer, moe = glm
    wl = gen.GLM_T256
    x, ids, w, outl = gen.make_inputs(wl)
    note(f"{wl.name}: run")
    got = call(moe, x, ids, w)
    assert moe.status() == pkg.MOE_OK
    counts, offsets, perm, inv = pkg.moe_fp8_prefill_debug_plan(moe.handle, wl.E, wl.T * wl.k)
    c, o, p, i, bad = oracle.plan(ids, wl.E)
    assert bad == 0 and np.array_equal(counts, c) and np.array_equal(offsets, o)
    assert np.array_equal(perm, p) and np.array_equal(inv, i)
    xq, sx = pkg.moe_fp8_prefill_debug_activations(moe.handle, wl.T, wl.H)
    q, s = oracle.quantize_rows(oracle.bf16_to_f32(x))
    assert np.array_equal(xq, q) and np.array_equal(sx.view(np.uint32), s.view(np.uint32))
    # every row against the oracle
    stagewise_on_sample(moe, layer, x, ids, w, wl.rho, got, np.arange(wl.T), wl.name)
    # repeated calls: identical hashes
    h0 = hashlib.sha256(got.tobytes()).hexdigest()
    for _ in range(2):
        assert hashlib.sha256(call(moe, x, ids, w).tobytes()).hexdigest() == h0
    # token permutation permutes rows bit for bit
    pi = np.random.default_rng(3).permutation(wl.T)
    assert np.array_equal(call(moe, x[pi], ids[pi], w[pi]), got[pi])


def test_glm_decode_t16(glm):
    """The W8A16 decode path on the full layer: a 16-token batch (the first
    16 rows of the T=256 inputs, outlier rows among them) against the
    oracle's W8A16 form, every row; and 256 rows through the decode path give
    the same bits for those 16 rows."""
    layer, moe = glm
    wl = gen.GLM_T256
    x, ids, w, outl = gen.make_inputs(wl)
    S = np.arange(16)
    note("glm decode T=16")
    out = moe.run_decode(dev_bf16(x[S]), dev(ids[S]), dev(w[S]))
    torch.cuda.synchronize()
    got = out_to_np(out)
    assert moe.status() == pkg.MOE_OK
    ref = oracle.forward_a16(layer, x[S], ids[S], w[S], wl.rho, oracle.OUT_BF16)
    assert_rows_close(got, ref, tol=TOL, what="glm decode T=16")
    big = moe.run_decode(dev_bf16(x), dev(ids), dev(w))
    torch.cuda.synchronize()
    assert np.array_equal(out_to_np(big)[S], got)


def test_glm_t4096(glm):
    layer, moe = glm
    wl = gen.GLM_T4096
    x, ids, w, outl = gen.make_inputs(wl)
    note(f"{wl.name}: run")
    got = call(moe, x, ids, w)
    counts, offsets, perm, inv = pkg.moe_fp8_prefill_debug_plan(moe.handle, wl.E, wl.T * wl.k)
    c, o, p, i, bad = oracle.plan(ids, wl.E)
    assert np.array_equal(counts, c) and np.array_equal(perm, p) and np.array_equal(inv, i)
    S = tile_kind_rows(ids, wl.E, outl)
    stagewise_on_sample(moe, layer, x, ids, w, wl.rho, got, S, wl.name)
    # a row alone gives the same bits as inside the 4096-row call
    for t in S[:4]:
        alone = call(moe, x[t:t + 1], ids[t:t + 1], w[t:t + 1])
        assert np.array_equal(alone[0], got[t]), t


def test_glm_t8192_zipf_chunking(glm):
    layer, moe = glm
    wl = gen.GLM_T8192_ZIPF
    x, ids, w, outl = gen.make_inputs(wl)
    note(f"{wl.name}: one call")
    one = call(moe, x, ids, w)
    counts, offsets, perm, inv = pkg.moe_fp8_prefill_debug_plan(moe.handle, wl.E, wl.T * wl.k)
    c, o, p, i, bad = oracle.plan(ids, wl.E)
    assert np.array_equal(counts, c) and np.array_equal(perm, p) and np.array_equal(inv, i)
    assert (counts == 0).sum() >= 8 and counts.max() > 4096
    S = tile_kind_rows(ids, wl.E, outl)
    stagewise_on_sample(moe, layer, x, ids, w, wl.rho, one, S, wl.name)
    for splits in ((4096, 8192), (4102, 8192), (1, 8192)):
        note(f"{wl.name}: calls split at {splits[0]}")
        parts, a = [], 0
        for b in splits:
            parts.append(call(moe, x[a:b], ids[a:b], w[a:b]))
            a = b
        assert np.array_equal(np.concatenate(parts), one), splits


@pytest.mark.parametrize("wl", [gen.SLICE_T16, gen.SLICE_T64, gen.SLICE_T1024], ids=lambda w: w.name)
def test_slice_layer(wl):
    note(f"{wl.name}: layer + run")
    layer = gen.make_layer(wl.E, wl.H, wl.I, seed=wl.seed)
    x, ids, w, outl = gen.make_inputs(wl)
    moe = pkg.MoeFp8Prefill(layer, wl.k, routed_scale=wl.rho, out_dtype=pkg.MOE_DTYPE_BF16)
    try:
        got = call(moe, x, ids, w)
        counts, offsets, perm, inv = pkg.moe_fp8_prefill_debug_plan(moe.handle, wl.E, wl.T * wl.k)
        c, o, p, i, bad = oracle.plan(ids, wl.E)
        assert np.array_equal(counts, c) and np.array_equal(perm, p) and np.array_equal(inv, i)
        S = np.arange(wl.T)  # every row
        stagewise_on_sample(moe, layer, x, ids, w, wl.rho, got, S, wl.name)
    finally:
        moe.close()


def test_glm_run_logits_t4096(glm):
    """The GLM layer from router logits (uniform draws, sigmoid top-8): the
    on-device router's ids equal the oracle's, and run_logits() equals run()
    on the routed ids and weights, bit for bit."""
    layer, moe = glm
    wl = gen.GLM_T4096
    x, _ = gen.make_tokens(wl.T, wl.H, wl.seed, wl.outlier_frac)
    logits = gen.make_logits(wl.T, wl.E, wl.route, wl.seed)
    note(f"{wl.name}: run_logits")
    xd, ld = dev_bf16(x), dev(logits)
    got = moe.run_logits(xd, ld, pkg.MOE_ROUTER_SIGMOID)
    ids_d, w_d = moe.route(ld, pkg.MOE_ROUTER_SIGMOID)
    ref = moe.run(xd, ids_d, w_d)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
    ids_o, w_o = oracle.route(logits, wl.k, oracle.ROUTE_SIGMOID)
    assert np.array_equal(ids_d.cpu().numpy(), ids_o)
    assert np.allclose(w_d.cpu().numpy(), w_o, rtol=8e-6, atol=1e-12)
