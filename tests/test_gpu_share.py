"""Load-time share of a wider checkpoint's intermediate dimension (GPU).

A handle built with share=(offset, length) keeps gate/up rows and down
columns [offset, offset+length) of the arrays; an unaligned offset makes
the load requantise every 128x128 block of the share.  The stored weights
(read back in the canonical layout) must equal the oracle's share bit for
bit (the codes are decided by FP32 values computed the same way on both
sides), for host and device sources and for a streamed slot; the layer on
the share must match the oracle on the oracle's share, stage by stage.
"""
import numpy as np
import pytest
import torch

import fp8_blockwise_routed_amd as pkg
import gen
import oracle
from gpu_util import compare_with_oracle, note, run

pytestmark = pytest.mark.gpu

E, K, H, I_FULL = 4, 2, 256, 384
SHARES = [(192, 192), (128, 256), (64, 100), (0, 192), (300, 84)]


def full_layer(seed=7):
    return gen.make_layer(E, H, I_FULL, seed=seed)


def assert_stored_equals(moe, ref, what):
    for e in range(E):
        got = pkg.moe_fp8_prefill_debug_unpack(moe.handle, e, H, ref.I)
        for key in ("gate", "up", "down"):
            assert np.array_equal(got[key], getattr(ref, key)[e]), (what, e, key)
        for key in ("gate_scale", "up_scale", "down_scale"):
            assert np.array_equal(got[key].view(np.uint32), getattr(ref, key)[e].view(np.uint32)), (what, e, key)


@pytest.mark.parametrize("share", SHARES, ids=[f"{o}+{n}" for o, n in SHARES])
def test_share_weights_match_oracle(share):
    layer = full_layer()
    ref = oracle.slice_layer(layer, *share)
    note(f"share {share}: host source")
    moe = pkg.MoeFp8Prefill(layer, K, share=share)
    try:
        assert_stored_equals(moe, ref, f"host {share}")
    finally:
        moe.close()
    note(f"share {share}: device source")
    dl = gen.Layer(E, H, I_FULL, *(torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in (
        layer.gate, layer.up, layer.down, layer.gate_scale, layer.up_scale, layer.down_scale)))
    moe = pkg.MoeFp8Prefill(dl, K, share=share, on_device=True)
    try:
        assert_stored_equals(moe, ref, f"device {share}")
    finally:
        moe.close()
    note(f"share {share}: streamed slot")
    sm = pkg.StreamedMoeFp8Prefill(layer, K, n_slots=1, share=share)
    try:
        sm.stage(0, layer)
        sm.select(0)
        torch.cuda.synchronize()
        assert_stored_equals(sm, ref, f"streamed {share}")
    finally:
        sm.close()


@pytest.mark.parametrize("share", [(192, 192), (64, 100)], ids=["192+192", "64+100"])
def test_layer_on_a_share(share):
    layer = full_layer(seed=8)
    ref = oracle.slice_layer(layer, *share)
    T = 80
    x, _ = gen.make_tokens(T, H, seed=8, outlier_frac=0.05)
    ids, w = gen.make_routing(T, E, K, gen.ROUTE_SIGMOID_NORMAL, seed=8)
    note(f"layer on share {share}")
    moe = pkg.MoeFp8Prefill(layer, K, routed_scale=2.5, out_dtype=pkg.MOE_DTYPE_F32, share=share)
    try:
        got = run(moe, x, ids, w)
        compare_with_oracle(moe, ref, x, ids, w, 2.5, got, what=f"share {share}")
    finally:
        moe.close()


def test_share_rejects():
    layer = full_layer()
    d, keep = pkg.make_desc(layer, K, share=(300, 100))      # past the end
    assert pkg.moe_fp8_prefill_validate(d) == pkg.MOE_ERR_INVALID_ARG
    d, keep = pkg.make_desc(layer, K, share=(0, 192))
    d.inter_full = 0
    d.inter_offset = 64                                        # offset without a share
    assert pkg.moe_fp8_prefill_validate(d) == pkg.MOE_ERR_INVALID_ARG
