"""Planted mistakes in the oracle must turn at least one pin red (CPU only).

Each fault is a plausible slip in the oracle (a wrong index, a dropped term, a
wrong sign, a transposed operand, a wrong rounding); the pins listed for it
must catch it.
"""
import pytest

import oracle
import pins

CAUGHT_BY = {
    "weight_scale_index": ["ffn_vs_bruteforce", "integer_exact_gate_up"],
    "drop_last_kblock": ["ffn_vs_bruteforce", "integer_exact_gate_up"],
    "unstable_plan": ["plan_vs_numpy"],
    "silu_clamp": ["ffn_vs_bruteforce"],
    "pad_garbage": ["ffn_vs_bruteforce", "integer_exact_gate_up"],
    "nan_code_is_nan": ["decode_golden", "decode_structure"],
    "group_64": ["quantize_vs_torch"],
    "down_scale_transposed": ["ffn_vs_bruteforce"],
    "encode_truncate": ["encode_vs_torch", "encode_vs_nearest_search"],
    "drop_rho": ["ffn_vs_bruteforce"],
    "silu_sign": ["ffn_vs_bruteforce", "activation_from_gu"],
    "gate_up_swap": ["ffn_vs_bruteforce", "activation_from_gu"],
    "route_tie_high": ["route_ids_vs_sort", "route_special_rows"],
    "route_all_experts": ["route_weights_vs_scipy", "route_special_rows"],
    "shared_inside_rho": ["shared_vs_bruteforce", "shared_composition"],
    "slice_scale_block": ["slice_requant_vs_torch", "slices_add_up"],
    "a16_h_truncate": ["a16_activation_from_gu", "a16_vs_bruteforce"],
}


@pytest.mark.parametrize("fault", sorted(CAUGHT_BY))
def test_fault_is_caught(fault):
    oracle.set_fault(fault)
    try:
        results = {name: pins.ALL_PINS[name]()[0] for name in CAUGHT_BY[fault]}
    finally:
        oracle.set_fault("none")
    assert not all(results.values()), f"fault {fault} slipped past {results}"


def test_every_fault_listed():
    assert set(CAUGHT_BY) == set(oracle.FAULTS) - {"none"}
