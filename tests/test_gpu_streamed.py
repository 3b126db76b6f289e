"""Streamed layer slots on the GPU (GPU).

A handle with two device weight slots that stage() refills from host
memory: every pass must equal, bit for bit, the same pass on a handle whose
weights were uploaded by create(); stage() must wait for the queued passes
that still read its slot (stream-ordered reuse); misuse and a staging
failure are refused (fail closed).
"""
import numpy as np
import pytest
import torch

import fp8_blockwise_routed_amd as pkg
import gen
from gpu_util import dev, dev_bf16, note, out_to_np

pytestmark = pytest.mark.gpu

E, K, H, I = 6, 2, 512, 192


def layers(n, seed0=10):
    return [gen.make_layer(E, H, I, seed=seed0 + i) for i in range(n)]


def pinned(layer):
    """The layer's arrays copied into page-locked host tensors."""
    out = {}
    for name in ("gate", "up", "down", "gate_scale", "up_scale", "down_scale"):
        a = getattr(layer, name)
        t = torch.empty(a.shape, dtype=torch.uint8 if a.dtype == np.uint8 else torch.float32, pin_memory=True)
        t.numpy()[...] = a
        out[name] = t
    return gen.Layer(layer.E, layer.H, layer.I, *(out[n] for n in ("gate", "up", "down", "gate_scale",
                                                                   "up_scale", "down_scale")))


def reference(layer, x, ids, w):
    moe = pkg.MoeFp8Prefill(layer, K, routed_scale=2.5, out_dtype=pkg.MOE_DTYPE_F32)
    try:
        out = moe.run(dev_bf16(x), dev(ids), dev(w))
        torch.cuda.synchronize()
        return out_to_np(out)
    finally:
        moe.close()


def test_slots_match_resident_layers():
    note("streamed slots vs resident layers")
    T = 300
    x, _ = gen.make_tokens(T, H, seed=1)
    ids, w = gen.make_routing(T, E, K, gen.ROUTE_SIGMOID_NORMAL, seed=1)
    ls = layers(4)
    refs = [reference(l, x, ids, w) for l in ls]
    hosts = [pinned(l) for l in ls]
    sm = pkg.StreamedMoeFp8Prefill(ls[0], K, n_slots=2, routed_scale=2.5, max_rows=128,
                                   out_dtype=pkg.MOE_DTYPE_F32)
    copy = torch.cuda.Stream()
    comp = torch.cuda.current_stream()
    try:
        xd, idd, wd = dev_bf16(x), dev(ids), dev(w)
        outs = [torch.empty((T, H), dtype=torch.float32, device="cuda") for _ in ls]
        sm.stage(0, hosts[0], stream=copy)
        for i in range(len(ls)):
            if i + 1 < len(ls):
                sm.stage((i + 1) % 2, hosts[i + 1], stream=copy)   # overlaps pass i
            sm.select(i % 2)
            sm.run(xd, idd, wd, out=outs[i], stream=comp)
        torch.cuda.synchronize()
        for i in range(len(ls)):
            assert np.array_equal(out_to_np(outs[i]).view(np.uint32), refs[i].view(np.uint32)), i
        assert sm.status() == pkg.MOE_OK
    finally:
        sm.close()


def test_stage_waits_for_passes_that_read_the_slot():
    """Queue several passes on slot 0, then immediately restage slot 0 with
    another layer on a second stream: the queued passes still see the old
    layer, and the next pass sees the new one."""
    note("stream-ordered slot reuse")
    T = 2048
    x, _ = gen.make_tokens(T, H, seed=2)
    ids, w = gen.make_routing(T, E, K, gen.ROUTE_SIGMOID_NORMAL, seed=2)
    la, lb = layers(2, seed0=30)
    ra, rb = reference(la, x, ids, w), reference(lb, x, ids, w)
    ha, hb = pinned(la), pinned(lb)
    sm = pkg.StreamedMoeFp8Prefill(la, K, n_slots=1, routed_scale=2.5, out_dtype=pkg.MOE_DTYPE_F32)
    copy = torch.cuda.Stream()
    comp = torch.cuda.current_stream()
    try:
        xd, idd, wd = dev_bf16(x), dev(ids), dev(w)
        sm.stage(0, ha, stream=copy)
        sm.select(0)
        first = [sm.run(xd, idd, wd, stream=comp) for _ in range(4)]
        sm.stage(0, hb, stream=copy)           # no host synchronisation before
        second = sm.run(xd, idd, wd, stream=comp)
        torch.cuda.synchronize()
        for o in first:
            assert np.array_equal(out_to_np(o).view(np.uint32), ra.view(np.uint32))
        assert np.array_equal(out_to_np(second).view(np.uint32), rb.view(np.uint32))
    finally:
        sm.close()


def test_streamed_misuse_and_fail_closed():
    la, = layers(1, seed0=50)
    sm = pkg.StreamedMoeFp8Prefill(la, K, n_slots=1, out_dtype=pkg.MOE_DTYPE_F32)
    try:
        x = dev_bf16(gen.make_tokens(8, H)[0])
        ids, w = gen.make_routing(8, E, K, gen.ROUTE_SIGMOID_NORMAL)
        out = torch.empty((8, H), dtype=torch.float32, device="cuda")
        # nothing staged yet
        assert pkg.moe_fp8_prefill_run(sm.handle, x, dev(ids), dev(w), 8, out) == pkg.MOE_ERR_INVALID_ARG
        assert pkg.moe_fp8_prefill_select_slot(sm.handle, 1) == pkg.MOE_ERR_INVALID_ARG
        assert pkg.moe_fp8_prefill_stage(sm.handle, 1, la.gate, la.up, la.down, la.gate_scale,
                                         la.up_scale, la.down_scale) == pkg.MOE_ERR_INVALID_ARG
        sm.stage(0, la)
        sm.select(0)
        assert pkg.moe_fp8_prefill_run(sm.handle, x, dev(ids), dev(w), 8, out) == pkg.MOE_OK
        pkg.moe_fp8_prefill_debug_inject_failure(sm.handle)
        assert pkg.moe_fp8_prefill_stage(sm.handle, 0, la.gate, la.up, la.down, la.gate_scale,
                                         la.up_scale, la.down_scale) == pkg.MOE_ERR_DEVICE
        assert pkg.moe_fp8_prefill_run(sm.handle, x, dev(ids), dev(w), 8, out) == pkg.MOE_ERR_FAILED_STATE
        assert pkg.moe_fp8_prefill_select_slot(sm.handle, 0) == pkg.MOE_ERR_FAILED_STATE
    finally:
        sm.close()
    # a resident handle has no slots
    moe = pkg.MoeFp8Prefill(la, K)
    try:
        assert pkg.moe_fp8_prefill_select_slot(moe.handle, 0) == pkg.MOE_ERR_INVALID_ARG
        assert pkg.moe_fp8_prefill_stage(moe.handle, 0, la.gate, la.up, la.down, la.gate_scale,
                                         la.up_scale, la.down_scale) == pkg.MOE_ERR_INVALID_ARG
    finally:
        moe.close()
