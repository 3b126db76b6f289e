"""The on-device top-k router against the oracle's router (GPU).

Expert ids are compared bit for bit (the decision is taken on the same FP32
logits on both sides); weights, computed in FP32 on the GPU and FP64 in the
oracle, within a relative 8e-6 (one expf and a k-term FP32 sum and divide).
Covers ties, -inf (masked experts), NaN, no-mass rows, E not a multiple of 64,
E = 1024 with k = 64, and run_logits() against run() on the routed ids.
"""
import numpy as np
import pytest
import torch

import fp8_blockwise_routed_amd as pkg
import gen
import oracle
from gpu_util import compare_with_oracle, dev, dev_bf16, note, out_to_np

pytestmark = pytest.mark.gpu

W_RTOL, W_ATOL = 8e-6, 1e-12


def special_logits(T, E, seed):
    rng = np.random.default_rng(seed)
    l = rng.standard_normal((T, E)).astype(np.float32)
    l[1, : E // 2] = 0.75                      # long tie
    l[2, :] = -0.0
    l[2, ::3] = 0.0                            # +0 and -0 are equal
    l[3, 1::2] = -np.inf                       # masked experts
    l[4, 0] = np.nan
    l[5, :] = -np.inf                          # no mass
    l[6, E - 1] = np.inf
    l[7, :] = np.nan                           # nothing but NaN
    return l


def route_both(moe, logits, kind):
    ids_d, w_d = moe.route(dev(logits), kind)
    torch.cuda.synchronize()
    ids_o, w_o = oracle.route(logits, moe.k, kind)
    return ids_d.cpu().numpy(), w_d.cpu().numpy(), ids_o, w_o


def assert_routes_equal(ids, w, ids_o, w_o, what):
    assert np.array_equal(ids, ids_o), f"{what}: ids differ in {(ids != ids_o).any(axis=1).sum()} rows"
    nan = np.isnan(w_o)
    assert np.array_equal(np.isnan(w), nan), f"{what}: NaN weights differ"
    ok = np.abs(w[~nan] - w_o[~nan]) <= W_RTOL * np.abs(w_o[~nan]) + W_ATOL
    assert ok.all(), f"{what}: weight off by {np.max(np.abs(w[~nan] - w_o[~nan]))}"


def tiny_handle(E, k, H=256, I=128):
    return pkg.MoeFp8Prefill(gen.make_layer(E, H, I, e_begin=0, e_end=E), k, max_rows=256)


@pytest.mark.parametrize("E,k", [(8, 2), (23, 4), (100, 8), (256, 8), (1024, 64)])
@pytest.mark.parametrize("kind", [pkg.MOE_ROUTER_SOFTMAX, pkg.MOE_ROUTER_SIGMOID])
def test_router_matches_oracle(E, k, kind):
    note(f"router E={E} k={k} kind={kind}")
    moe = tiny_handle(E, k)
    try:
        for T, seed in ((1, 0), (97, 1), (513, 2)):
            l = special_logits(max(T, 8), E, seed)[:T]
            ids, w, ids_o, w_o = route_both(moe, l, kind)
            assert_routes_equal(ids, w, ids_o, w_o, f"E={E} k={k} T={T}")
        # T = 0 is a no-op
        assert pkg.moe_fp8_prefill_route(moe.handle, 0, kind, 0, 0, 0) == pkg.MOE_OK
    finally:
        moe.close()


@pytest.mark.parametrize("kind,route,masked,T", [
    (pkg.MOE_ROUTER_SIGMOID, gen.ROUTE_SIGMOID_NORMAL, 0, 256),
    (pkg.MOE_ROUTER_SIGMOID, gen.ROUTE_SIGMOID_UNIFORM, 0, 4096),
    (pkg.MOE_ROUTER_SIGMOID, gen.ROUTE_ZIPF, 8, 8192),
], ids=["sigmoid_t256", "uniform_t4096", "zipf_t8192"])
def test_router_on_workload_logits(kind, route, masked, T):
    """The GLM layer's router shapes (E=256, top-8) on the workloads' logits;
    the generator's own FP64 routing must agree too."""
    note(f"router workload logits route={route} T={T}")
    moe = tiny_handle(256, 8)
    try:
        l = gen.make_logits(T, 256, route, 0, masked)
        ids, w, ids_o, w_o = route_both(moe, l, kind)
        assert_routes_equal(ids, w, ids_o, w_o, f"route={route} T={T}")
        ids_g, _ = gen.make_routing(T, 256, 8, route, 0, masked)
        assert np.array_equal(ids, ids_g)
    finally:
        moe.close()


def test_router_rejects():
    moe = tiny_handle(128, 65)
    try:
        l = dev(np.zeros((4, 128), np.float32))
        ids = torch.empty((4, 65), dtype=torch.int32, device="cuda")
        w = torch.empty((4, 65), dtype=torch.float32, device="cuda")
        assert pkg.moe_fp8_prefill_route(moe.handle, l, 0, 4, ids, w) == pkg.MOE_ERR_UNSUPPORTED
        x = dev_bf16(np.zeros((4, 256), np.uint16))
        out = torch.empty((4, 256), dtype=torch.bfloat16, device="cuda")
        assert pkg.moe_fp8_prefill_run_logits(moe.handle, x, l, 0, 4, out) == pkg.MOE_ERR_UNSUPPORTED
    finally:
        moe.close()
    moe = tiny_handle(8, 2)
    try:
        l = dev(np.zeros((4, 8), np.float32))
        ids = torch.empty((4, 2), dtype=torch.int32, device="cuda")
        w = torch.empty((4, 2), dtype=torch.float32, device="cuda")
        assert pkg.moe_fp8_prefill_route(moe.handle, l, 2, 4, ids, w) == pkg.MOE_ERR_INVALID_ARG
        assert pkg.moe_fp8_prefill_route(moe.handle, 0, 0, 4, ids, w) == pkg.MOE_ERR_INVALID_ARG
        assert moe.status() == pkg.MOE_OK  # rejections leave the handle usable
    finally:
        moe.close()


@pytest.mark.parametrize("E,k,H,I,T,kind,rho", [
    (8, 2, 256, 128, 64, pkg.MOE_ROUTER_SOFTMAX, 1.0),
    (6, 3, 512, 192, 300, pkg.MOE_ROUTER_SIGMOID, 2.5),
])
def test_run_logits(E, k, H, I, T, kind, rho):
    """run_logits() = run() on the routed ids and weights, bit for bit, across
    internal passes (max_rows 128 < T); and the staged oracle comparison on
    the oracle's own routing of the same logits."""
    note(f"run_logits E={E} k={k} T={T}")
    layer = gen.make_layer(E, H, I)
    x, _ = gen.make_tokens(T, H, outlier_frac=0.02)
    route = gen.ROUTE_SOFTMAX if kind == pkg.MOE_ROUTER_SOFTMAX else gen.ROUTE_SIGMOID_NORMAL
    l = gen.make_logits(T, E, route)
    moe = pkg.MoeFp8Prefill(layer, k, routed_scale=rho, max_rows=128, out_dtype=pkg.MOE_DTYPE_F32)
    try:
        xd, ld = dev_bf16(x), dev(l)
        got = moe.run_logits(xd, ld, kind)
        ids_d, w_d = moe.route(ld, kind)
        ref = moe.run(xd, ids_d, w_d)
        torch.cuda.synchronize()
        assert torch.equal(got, ref)
        ids_o, w_o = oracle.route(l, k, kind)
        assert np.array_equal(ids_d.cpu().numpy(), ids_o)
        # one pass holding every row, so the debug views cover the whole call
        moe_all = pkg.MoeFp8Prefill(layer, k, routed_scale=rho, max_rows=T, out_dtype=pkg.MOE_DTYPE_F32)
        try:
            got_all = moe_all.run_logits(xd, ld, kind)
            torch.cuda.synchronize()
            assert torch.equal(got_all, got)
            compare_with_oracle(moe_all, layer, x, ids_o, w_d.cpu().numpy(), rho, out_to_np(got_all),
                                what=f"run_logits E={E}")
        finally:
            moe_all.close()
    finally:
        moe.close()
