"""The W8A16 decode path (moe_fp8_prefill_run_decode) vs the oracle's W8A16
form of the layer (GPU).

Covers: per-row output vs oracle.forward_a16 (relative L2 <= 2e-2) on
layers whose experts get from 0 to several hundred rows (tiles of all three
plan lists taken 16 rows at a time, ragged tails), I=192 zero padding, the
shared-expert slot and the clamped SiLU; row bits independent of the
neighbours and of the pass split (1024-row passes); the method is not the
prefill path's (W8A8) and each matches its own oracle form.
"""
import numpy as np
import pytest
import torch

import fp8_blockwise_routed_amd as pkg
import gen
import oracle
from gpu_util import TOL, assert_rows_close, dev, dev_bf16, note, out_to_np, rel_l2_rows, run

pytestmark = pytest.mark.gpu

# (E, k, H, I, T, route, rho, outlier_frac)
CASES = [
    ("tiny", (8, 2, 256, 128, 64, gen.ROUTE_SOFTMAX, 1.0, 0.0)),
    ("decode_t1", (16, 4, 512, 256, 1, gen.ROUTE_SIGMOID_NORMAL, 2.5, 0.0)),
    ("pad192", (6, 3, 512, 192, 50, gen.ROUTE_SIGMOID_NORMAL, 2.5, 0.05)),
    ("many_rows", (4, 2, 256, 256, 600, gen.ROUTE_SIGMOID_UNIFORM, 2.5, 0.01)),
    ("odd_blocks", (3, 2, 384, 320, 90, gen.ROUTE_SIGMOID_UNIFORM, 2.5, 0.01)),
    # the flat down variants over several K steps: Ip/128 = 4 (four blocks in
    # flight) and Ip/128 = 6 (two in flight, three ring turns per unit), ~100
    # rows per expert so workgroups run several 16-row units
    ("flat4_i512", (6, 2, 256, 512, 300, gen.ROUTE_SIGMOID_UNIFORM, 2.5, 0.01)),
    ("flat2_i768", (5, 2, 384, 768, 300, gen.ROUTE_SIGMOID_UNIFORM, 2.5, 0.01)),
]


def make_case(spec, seed=0):
    E, k, H, I, T, route, rho, of = spec
    layer = gen.make_layer(E, H, I, seed=seed)
    x, _ = gen.make_tokens(T, H, seed=seed, outlier_frac=of)
    ids, w = gen.make_routing(T, E, k, route, seed=seed)
    return layer, x, ids, w, rho


def decode(moe, x, ids, w):
    out = moe.run_decode(dev_bf16(x), dev(ids), dev(w))
    torch.cuda.synchronize()
    return out_to_np(out)


@pytest.mark.parametrize("name,spec", CASES)
@pytest.mark.parametrize("out_dtype", [pkg.MOE_DTYPE_BF16, pkg.MOE_DTYPE_F32])
def test_decode_vs_oracle(name, spec, out_dtype):
    layer, x, ids, w, rho = make_case(spec)
    ref = oracle.forward_a16(layer, x, ids, w, rho, oracle.OUT_BF16 if out_dtype == pkg.MOE_DTYPE_BF16 else oracle.OUT_F32)
    note(f"decode {name} out_dtype={out_dtype}")
    moe = pkg.MoeFp8Prefill(layer, spec[1], routed_scale=rho, out_dtype=out_dtype)
    try:
        got = decode(moe, x, ids, w)
        assert moe.status() == pkg.MOE_OK
    finally:
        moe.close()
    assert_rows_close(got, ref, TOL, f"decode {name}")
    # far tighter than the bar in practice: FP32 sum order and the odd BF16
    # rounding of h near a tie are the only differences
    assert float(rel_l2_rows(got, ref).max()) < 2e-3


def test_decode_rows_independent_and_pass_split():
    """A row's bits do not depend on its neighbours or on the 1024-row passes:
    1100 rows in one call (passes of 1024 + 76) equal calls of 550 + 550 and
    of single rows."""
    spec = (8, 2, 256, 128, 1100, gen.ROUTE_SIGMOID_NORMAL, 2.5, 0.01)
    layer, x, ids, w, rho = make_case(spec, seed=3)
    note("decode invariance 1100 rows")
    moe = pkg.MoeFp8Prefill(layer, 2, routed_scale=rho, out_dtype=pkg.MOE_DTYPE_F32, max_rows=2048)
    try:
        full = decode(moe, x, ids, w)
        halves = np.concatenate([decode(moe, x[:550], ids[:550], w[:550]),
                                 decode(moe, x[550:], ids[550:], w[550:])])
        singles = np.concatenate([decode(moe, x[i:i + 1], ids[i:i + 1], w[i:i + 1]) for i in (0, 1, 1023, 1024, 1099)])
    finally:
        moe.close()
    assert np.array_equal(full.view(np.uint32), halves.view(np.uint32))
    assert np.array_equal(full[[0, 1, 1023, 1024, 1099]].view(np.uint32), singles.view(np.uint32))


@pytest.mark.parametrize("name,spec", [c for c in CASES if c[0].startswith("flat")])
def test_decode_flat_pass_split(name, spec):
    """The flat down variants: a row's bits do not depend on the pass split
    (300 rows in one call = 150 + 150 = passes of 64 rows)."""
    layer, x, ids, w, rho = make_case(spec, seed=4)
    note(f"decode pass split {name}")
    moe = pkg.MoeFp8Prefill(layer, spec[1], routed_scale=rho, out_dtype=pkg.MOE_DTYPE_F32)
    small = pkg.MoeFp8Prefill(layer, spec[1], routed_scale=rho, out_dtype=pkg.MOE_DTYPE_F32, max_rows=64)
    try:
        full = decode(moe, x, ids, w)
        halves = np.concatenate([decode(moe, x[:150], ids[:150], w[:150]),
                                 decode(moe, x[150:], ids[150:], w[150:])])
        passes = decode(small, x, ids, w)
    finally:
        moe.close()
        small.close()
    assert np.array_equal(full.view(np.uint32), halves.view(np.uint32))
    assert np.array_equal(full.view(np.uint32), passes.view(np.uint32))


def test_decode_is_its_own_method():
    """Decode (W8A16) and run (W8A8) each match their own oracle form and
    differ from each other by about the E4M3 quantisation error."""
    layer, x, ids, w, rho = make_case(CASES[2][1])
    note("decode vs prefill")
    moe = pkg.MoeFp8Prefill(layer, 3, routed_scale=rho, out_dtype=pkg.MOE_DTYPE_F32)
    try:
        dec = decode(moe, x, ids, w)
        pre = run(moe, x, ids, w)
    finally:
        moe.close()
    ref16 = oracle.forward_a16(layer, x, ids, w, rho, oracle.OUT_F32)
    ref8 = oracle.forward(layer, x, ids, w, rho, oracle.OUT_F32)
    assert float(rel_l2_rows(dec, ref16).max()) < 2e-3
    assert float(rel_l2_rows(pre, ref8).max()) < TOL
    between = float(rel_l2_rows(dec, pre).mean())
    assert 1e-2 < between < 2e-1, between


def test_decode_shared_and_clamped():
    """The shared-expert slot and the clamped SiLU go through the decode path
    as through run()."""
    E, k, H, I, T = 6, 2, 256, 128, 40
    layer = gen.make_layer(E + 1, H, I, seed=5)
    x, _ = gen.make_tokens(T, H, seed=5, outlier_frac=0.0)
    ids, w = gen.make_routing(T, E, k, gen.ROUTE_SIGMOID_NORMAL, seed=5)
    ids_all = np.concatenate([ids, np.full((T, 1), E, np.int32)], axis=1)
    w_all = np.concatenate([w, np.ones((T, 1), np.float32)], axis=1)
    oracle.set_activation_limit(1.5)
    try:
        ref = oracle.forward_a16(layer, x, ids_all, w_all, 2.5, oracle.OUT_F32, n_shared=1)
    finally:
        oracle.set_activation_limit(0.0)
    note("decode shared + clamped")
    moe = pkg.MoeFp8Prefill(layer, k, routed_scale=2.5, out_dtype=pkg.MOE_DTYPE_F32, shared_experts=1,
                            activation_limit=1.5)
    try:
        got = decode(moe, x, ids, w)
    finally:
        moe.close()
    assert float(rel_l2_rows(got, ref).max()) < 2e-3


def test_decode_empty_and_null():
    layer, x, ids, w, rho = make_case(CASES[0][1])
    moe = pkg.MoeFp8Prefill(layer, 2, routed_scale=rho)
    try:
        out = torch.empty((1, layer.H), dtype=torch.bfloat16, device="cuda")
        assert pkg.moe_fp8_prefill_run_decode(moe.handle, dev_bf16(x[:1]), dev(ids[:1]), dev(w[:1]), 0, out) == pkg.MOE_OK
        assert pkg.moe_fp8_prefill_run_decode(moe.handle, None, None, None, 1, None) == pkg.MOE_ERR_INVALID_ARG
    finally:
        moe.close()
    assert pkg.moe_fp8_prefill_run_decode(0, None, None, None, 1, None) == pkg.MOE_ERR_INVALID_ARG
