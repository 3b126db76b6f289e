"""The always-on shared-expert slot on the GPU (GPU).

A layer of E routed experts plus one shared expert (the arrays' last): every
token gets a (k+1)-th slot on it, computed in the same grouped GEMMs and
added after the routed sum is scaled.  Checked against the oracle with the
shared slot (plan bit for bit over k+1 slots, staged output comparison), and
as a composition: the layer with the shared slot equals, bit for bit, the
routed layer plus the shared expert run on its own (FP32 output, one add).
"""
import numpy as np
import pytest
import torch

import fp8_blockwise_routed_amd as pkg
import gen
import oracle
from gpu_util import compare_with_oracle, dev, dev_bf16, note, out_to_np, run, with_shared_slot

pytestmark = pytest.mark.gpu

CASES = [
    # name, (E routed, k, H, I, T, rho, route)
    ("pad192", (6, 3, 512, 192, 50, 2.5, gen.ROUTE_SIGMOID_NORMAL)),
    ("many_rows", (4, 2, 256, 256, 600, 1.0, gen.ROUTE_SIGMOID_UNIFORM)),
    ("slice_t64", (160, 8, 5120, 192, 64, 1.0, gen.ROUTE_SIGMOID_NORMAL)),
    # the most slots a token can have: every one of 256 experts plus the
    # shared one (257 slots per token in the combine)
    ("k256_all", (256, 256, 128, 128, 3, 1.0, gen.ROUTE_SIGMOID_NORMAL)),
]


def shared_case(spec, seed=0):
    E, k, H, I, T, rho, route = spec
    layer = gen.make_layer(E + 1, H, I, seed=seed)
    x, _ = gen.make_tokens(T, H, seed=seed, outlier_frac=0.02)
    if k <= 64:
        ids, w = gen.make_routing(T, E, k, route, seed=seed)
    else:  # beyond the generator's router: every token takes k distinct experts
        rng = np.random.default_rng(seed)
        ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
        w = rng.uniform(0.5, 1.5, size=(T, k)).astype(np.float32)
        w /= w.sum(axis=1, keepdims=True)
    return layer, x, ids, w, rho


@pytest.mark.parametrize("name,spec", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("out_dtype", [pkg.MOE_DTYPE_F32, pkg.MOE_DTYPE_BF16], ids=["f32", "bf16"])
def test_shared_slot_matches_oracle(name, spec, out_dtype):
    layer, x, ids, w, rho = shared_case(spec)
    E, k, T = spec[0], spec[1], spec[4]
    note(f"shared slot {name} out={out_dtype}")
    moe = pkg.MoeFp8Prefill(layer, k, routed_scale=rho, max_rows=T, out_dtype=out_dtype, shared_experts=1)
    try:
        got = run(moe, x, ids, w)
        assert moe.status() == pkg.MOE_OK
        ids_x, w_x = with_shared_slot(ids, w, E)
        counts, offsets, perm, inv = pkg.moe_fp8_prefill_debug_plan(moe.handle, E + 1, T * (k + 1))
        c, o, p, i, bad = oracle.plan(ids_x, E + 1)
        assert bad == 0 and counts[E] == T
        assert np.array_equal(counts, c) and np.array_equal(perm, p) and np.array_equal(inv, i)
        compare_with_oracle(moe, layer, x, ids_x, w_x, rho, got, what=f"shared {name}", n_shared=1)
    finally:
        moe.close()


def test_shared_slot_is_routed_plus_shared_expert():
    """Bit for bit: out(shared) = routed-only out + shared expert alone (FP32)."""
    E, k, H, I, T, rho = 5, 2, 384, 128, 137, 2.5
    layer = gen.make_layer(E + 1, H, I, seed=3)
    x, _ = gen.make_tokens(T, H, seed=3)
    ids, w = gen.make_routing(T, E, k, gen.ROUTE_SIGMOID_NORMAL, seed=3)
    ids[5, 0] = -1                       # a skip slot stays skipped
    note("shared composition")
    part = lambda a, lo, hi: a[lo:hi]
    routed = gen.Layer(E, H, I, *(part(a, 0, E) for a in (layer.gate, layer.up, layer.down, layer.gate_scale,
                                                        layer.up_scale, layer.down_scale)))
    shared = gen.Layer(1, H, I, *(part(a, E, E + 1) for a in (layer.gate, layer.up, layer.down,
                                                            layer.gate_scale, layer.up_scale,
                                                            layer.down_scale)))
    f32 = pkg.MOE_DTYPE_F32
    m_all = pkg.MoeFp8Prefill(layer, k, routed_scale=rho, out_dtype=f32, shared_experts=1, max_rows=64)
    m_r = pkg.MoeFp8Prefill(routed, k, routed_scale=rho, out_dtype=f32)
    m_s = pkg.MoeFp8Prefill(shared, 1, routed_scale=1.0, out_dtype=f32)
    try:
        got = run(m_all, x, ids, w)           # three internal passes
        r = run(m_r, x, ids, w)
        s_ = run(m_s, x, np.zeros((T, 1), np.int32), np.ones((T, 1), np.float32))
        assert np.array_equal((r + s_).view(np.uint32), got.view(np.uint32))
    finally:
        for m in (m_all, m_r, m_s):
            m.close()


def test_shared_slot_bad_ids_and_router():
    """A routed id equal to E (the shared expert's index) is a bad id; the
    shared slot itself is always planned.  run_logits routes over the E
    routed experts only."""
    E, k, H, I, T = 6, 2, 256, 128, 40
    layer = gen.make_layer(E + 1, H, I, seed=5)
    x, _ = gen.make_tokens(T, H, seed=5)
    ids, w = gen.make_routing(T, E, k, gen.ROUTE_SOFTMAX, seed=5)
    moe = pkg.MoeFp8Prefill(layer, k, out_dtype=pkg.MOE_DTYPE_F32, shared_experts=1)
    try:
        bad = ids.copy()
        bad[7, 1] = E
        got_bad = run(moe, x, bad, w)
        assert moe.status() == pkg.MOE_ERR_BAD_EXPERT_ID
        skip = ids.copy()
        skip[7, 1] = -1
        assert np.array_equal(got_bad.view(np.uint32), run(moe, x, skip, w).view(np.uint32))
        assert moe.status() == pkg.MOE_OK
        logits = gen.make_logits(T, E, gen.ROUTE_SOFTMAX, 5)
        ld = dev(logits)
        got = moe.run_logits(dev_bf16(x), ld, pkg.MOE_ROUTER_SOFTMAX)
        ids_d, w_d = moe.route(ld, pkg.MOE_ROUTER_SOFTMAX)
        ref = moe.run(dev_bf16(x), ids_d, w_d)
        torch.cuda.synchronize()
        assert torch.equal(got, ref)
        assert np.array_equal(ids_d.cpu().numpy(), oracle.route(logits, k, oracle.ROUTE_SOFTMAX)[0])
    finally:
        moe.close()
