"""The C-ABI library on the host: it loads, exports every declared entry
point, and its pure-host calls (validate, sizes, strerror) behave (CPU only;
no call here touches a GPU)."""
import ctypes
import os
import re

import pytest

import fp8_blockwise_routed_amd as pkg
import gen

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                      "moe_fp8_prefill.h")


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(moe_fp8_prefill_\w+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    lib = pkg.load_library()
    names = declared_functions()
    assert len(names) >= 16
    for n in names:
        getattr(lib, n)
    assert set(names) == set(pkg.EXPORTED)


def _desc(**over):
    layer = gen.make_layer(8, 256, 128)
    d, keep = pkg.make_desc(layer, 2, max_rows=64)
    for k, v in over.items():
        setattr(d, k, v)
    return d, keep


def test_validate_accepts_the_configurations():
    for E, k, H, I in ((8, 2, 256, 128), (256, 8, 6144, 2048), (160, 8, 5120, 192)):
        layer = gen.Layer(E, H, I, *([None] * 6))
        fake = type("L", (), dict(E=E, H=H, I=I, gate=None))
        d = pkg.moe_fp8_prefill_desc(ctypes.sizeof(pkg.moe_fp8_prefill_desc), E, k, H, I, 8192,
                                     pkg.MOE_DTYPE_BF16, pkg.MOE_ACT_SILU_UNCLAMPED, 128, 2.5, 0,
                                     1, 1, 1, 1, 1, 1, None)
        assert pkg.moe_fp8_prefill_validate(d) == pkg.MOE_OK, (E, k, H, I)
        assert pkg.moe_fp8_prefill_workspace_bytes(d) > 0
    # the GLM layer's weights: 9.002 GiB of codes and scales
    d.num_experts, d.top_k, d.hidden, d.inter = 256, 8, 6144, 2048
    assert round(pkg.moe_fp8_prefill_weight_bytes(d) / 2 ** 30, 3) == 9.002


@pytest.mark.parametrize("field,value,code", [
    ("hidden", 200, pkg.MOE_ERR_UNSUPPORTED),          # H % 128 != 0
    ("top_k", 9, pkg.MOE_ERR_UNSUPPORTED),             # k > E
    ("top_k", 0, pkg.MOE_ERR_INVALID_ARG),
    ("num_experts", 0, pkg.MOE_ERR_INVALID_ARG),
    ("num_experts", 2000, pkg.MOE_ERR_UNSUPPORTED),
    ("inter", 0, pkg.MOE_ERR_INVALID_ARG),
    ("max_rows", 0, pkg.MOE_ERR_INVALID_ARG),
    ("block", 64, pkg.MOE_ERR_UNSUPPORTED),
    ("activation", 2, pkg.MOE_ERR_UNSUPPORTED),
    ("out_dtype", 5, pkg.MOE_ERR_UNSUPPORTED),
    ("routed_scale", float("nan"), pkg.MOE_ERR_INVALID_ARG),
    ("struct_size", 8, pkg.MOE_ERR_INVALID_ARG),
    ("gate", None, pkg.MOE_ERR_INVALID_ARG),
])
def test_validate_rejects(field, value, code):
    d, keep = _desc(**{field: value})
    assert pkg.moe_fp8_prefill_validate(d) == code
    assert pkg.moe_fp8_prefill_workspace_bytes(d) == -code


def test_validate_rejects_null():
    assert pkg.load_library().moe_fp8_prefill_validate(None) == pkg.MOE_ERR_INVALID_ARG


def test_create_rejects_before_allocating():
    """An invalid description is refused by create() without any GPU call."""
    d, keep = _desc(hidden=200)
    with pytest.raises(pkg.MoeError) as ei:
        pkg.moe_fp8_prefill_create(d)
    assert ei.value.code == pkg.MOE_ERR_UNSUPPORTED


def test_null_handle_calls():
    lib = pkg.load_library()
    assert lib.moe_fp8_prefill_run(None, None, None, None, 1, None, None) == pkg.MOE_ERR_INVALID_ARG
    assert lib.moe_fp8_prefill_run_decode(None, None, None, None, 1, None, None) == pkg.MOE_ERR_INVALID_ARG
    assert lib.moe_fp8_prefill_status(None) == pkg.MOE_ERR_INVALID_ARG
    assert lib.moe_fp8_prefill_set_timing(None, 1) == pkg.MOE_ERR_INVALID_ARG
    assert lib.moe_fp8_prefill_set_timing_stages(None, 1) == pkg.MOE_ERR_INVALID_ARG
    assert lib.moe_fp8_prefill_route(None, None, 0, 1, None, None, None) == pkg.MOE_ERR_INVALID_ARG
    assert lib.moe_fp8_prefill_run_logits(None, None, None, 0, 1, None, None) == pkg.MOE_ERR_INVALID_ARG
    assert lib.moe_fp8_prefill_stage(None, 0, None, None, None, None, None, None, None) == pkg.MOE_ERR_INVALID_ARG
    assert lib.moe_fp8_prefill_select_slot(None, 0) == pkg.MOE_ERR_INVALID_ARG
    h = ctypes.c_void_p()
    assert lib.moe_fp8_prefill_create_streamed(None, 2, ctypes.byref(h)) == pkg.MOE_ERR_INVALID_ARG
    assert h.value is None
    lib.moe_fp8_prefill_destroy(None)  # NULL-safe


def test_strerror_covers_all_codes():
    for c in range(8):
        assert pkg.moe_fp8_prefill_strerror(c) != "unknown error code"
    assert pkg.moe_fp8_prefill_strerror(99) == "unknown error code"


def test_shared_expert_field():
    d, keep = _desc()
    assert pkg.moe_fp8_prefill_validate(d) == pkg.MOE_OK
    base = pkg.moe_fp8_prefill_workspace_bytes(d)
    d.shared_experts = 1
    assert pkg.moe_fp8_prefill_validate(d) == pkg.MOE_OK
    assert pkg.moe_fp8_prefill_workspace_bytes(d) > base      # k+1 slots per row
    d.shared_experts = 2
    assert pkg.moe_fp8_prefill_validate(d) == pkg.MOE_ERR_UNSUPPORTED
    d.shared_experts = 1
    d.num_experts = 1024                                       # 1024 + 1 experts
    d.top_k = 2
    assert pkg.moe_fp8_prefill_validate(d) == pkg.MOE_ERR_UNSUPPORTED
    # a description built without the field (the size up to it) still validates
    d2, keep2 = _desc()
    d2.struct_size = pkg.moe_fp8_prefill_desc.shared_experts.offset
    assert pkg.moe_fp8_prefill_validate(d2) == pkg.MOE_OK
    d2.struct_size = pkg.moe_fp8_prefill_desc.activation_limit.offset
    assert pkg.moe_fp8_prefill_validate(d2) == pkg.MOE_OK
    d2.struct_size = 12
    assert pkg.moe_fp8_prefill_validate(d2) == pkg.MOE_ERR_INVALID_ARG


def test_clamped_activation_field():
    d, keep = _desc()
    d.activation = pkg.MOE_ACT_SILU_CLAMPED
    assert pkg.moe_fp8_prefill_validate(d) == pkg.MOE_ERR_INVALID_ARG   # limit 0
    d.activation_limit = 10.0
    assert pkg.moe_fp8_prefill_validate(d) == pkg.MOE_OK
    d.activation_limit = float("inf")
    assert pkg.moe_fp8_prefill_validate(d) == pkg.MOE_ERR_INVALID_ARG
    d.activation_limit = -1.0
    assert pkg.moe_fp8_prefill_validate(d) == pkg.MOE_ERR_INVALID_ARG
    d.activation = pkg.MOE_ACT_SILU_UNCLAMPED
    d.activation_limit = 10.0                                          # limit without the clamp
    assert pkg.moe_fp8_prefill_validate(d) == pkg.MOE_ERR_INVALID_ARG
    d.activation = 7
    d.activation_limit = 0.0
    assert pkg.moe_fp8_prefill_validate(d) == pkg.MOE_ERR_UNSUPPORTED


def test_share_fields():
    layer = gen.make_layer(4, 256, 384)
    d, keep = pkg.make_desc(layer, 2, share=(192, 192))
    assert pkg.moe_fp8_prefill_validate(d) == pkg.MOE_OK
    d, keep = pkg.make_desc(layer, 2, share=(300, 100))
    assert pkg.moe_fp8_prefill_validate(d) == pkg.MOE_ERR_INVALID_ARG
    d, keep = pkg.make_desc(layer, 2, share=(-1, 100))
    assert pkg.moe_fp8_prefill_validate(d) == pkg.MOE_ERR_INVALID_ARG
    d, keep = pkg.make_desc(layer, 2)
    d.inter_offset = 5
    assert pkg.moe_fp8_prefill_validate(d) == pkg.MOE_ERR_INVALID_ARG
    d.inter_offset = 0
    d.struct_size = pkg.moe_fp8_prefill_desc.inter_full.offset   # a caller without the fields
    assert pkg.moe_fp8_prefill_validate(d) == pkg.MOE_OK
