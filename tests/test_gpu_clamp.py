"""The clamped SiLU variant on the GPU (GPU).

MOE_ACT_SILU_CLAMPED with limit L caps the gate at L and clips up to [-L, L]
before silu(gate) * up.  Compared stage by stage with the oracle set to the
same limit, on the 1-subtile and the 256-row tile GEMMs; a limit chosen
below the layers' typical |gate| so the clamp is active; a huge limit gives
the unclamped bits.
"""
import numpy as np
import pytest

import fp8_blockwise_routed_amd as pkg
import gen
from gpu_util import compare_with_oracle, note, rel_l2_rows, run

pytestmark = pytest.mark.gpu

CASES = [
    # name, (E, k, H, I, T, rho, route, limit)
    ("few_rows", (8, 2, 256, 128, 64, 1.0, gen.ROUTE_SOFTMAX, 0.5)),
    ("pad192", (6, 3, 512, 192, 50, 2.5, gen.ROUTE_SIGMOID_NORMAL, 0.4)),
    ("many_rows", (4, 2, 256, 256, 600, 2.5, gen.ROUTE_SIGMOID_UNIFORM, 0.3)),
]


@pytest.mark.parametrize("name,spec", CASES, ids=[c[0] for c in CASES])
def test_clamped_silu_matches_oracle(name, spec):
    E, k, H, I, T, rho, route, L = spec
    layer = gen.make_layer(E, H, I)
    x, _ = gen.make_tokens(T, H, outlier_frac=0.02)
    ids, w = gen.make_routing(T, E, k, route)
    note(f"clamped SiLU {name} L={L}")
    moe = pkg.MoeFp8Prefill(layer, k, routed_scale=rho, max_rows=T, out_dtype=pkg.MOE_DTYPE_F32,
                            activation_limit=L)
    plain = pkg.MoeFp8Prefill(layer, k, routed_scale=rho, max_rows=T, out_dtype=pkg.MOE_DTYPE_F32)
    try:
        got = run(moe, x, ids, w)
        compare_with_oracle(moe, layer, x, ids, w, rho, got, what=f"clamped {name}", act_limit=L)
        unclamped = run(plain, x, ids, w)
        assert rel_l2_rows(got, unclamped).max() > 1e-2   # the clamp is active
    finally:
        moe.close()
        plain.close()


def test_huge_limit_is_unclamped():
    E, k, H, I, T = 5, 2, 384, 192, 90
    layer = gen.make_layer(E, H, I, seed=2)
    x, _ = gen.make_tokens(T, H, seed=2)
    ids, w = gen.make_routing(T, E, k, gen.ROUTE_SIGMOID_NORMAL, seed=2)
    a = pkg.MoeFp8Prefill(layer, k, out_dtype=pkg.MOE_DTYPE_F32, activation_limit=1e30)
    b = pkg.MoeFp8Prefill(layer, k, out_dtype=pkg.MOE_DTYPE_F32)
    try:
        assert np.array_equal(run(a, x, ids, w).view(np.uint32), run(b, x, ids, w).view(np.uint32))
    finally:
        a.close()
        b.close()
