"""A seeded sweep of random small layers, GPU path vs the oracle (GPU).

Each case draws E, top-k, H, I (not a multiple of 128 in most cases, so the
intermediate edge is zero-padded), T, the routing recipe, the routed scale
and the outlier share from a fixed seed, so the sweep reaches shapes the
named cases do not: single experts, top-k equal to E, one-row batches,
experts with rows on both sides of the 16- and 128-row tile limits, and
H / 128 and Ip / 128 odd and even.  Per case: the staged comparison with the
oracle (gate/up, every h code, y and the output from the kernel's h, the
plain per-row bound), and the same rows run again in passes of a random
smaller max_rows must give the same output bits.
"""
import numpy as np
import pytest

import fp8_blockwise_routed_amd as pkg
import gen
from gpu_util import compare_with_oracle, note, run

pytestmark = pytest.mark.gpu

ROUTES = (gen.ROUTE_SOFTMAX, gen.ROUTE_SIGMOID_NORMAL, gen.ROUTE_SIGMOID_UNIFORM, gen.ROUTE_ZIPF)


def sweep_cases(n=28, seed=20261203):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        E = int(rng.choice([1, 2, 3, 5, 8, 13, 24, 40]))
        k = int(rng.integers(1, min(E, 8) + 1))
        H = 128 * int(rng.integers(1, 13))
        I = int(rng.choice([int(rng.integers(1, 128)), int(rng.integers(129, 700)), 128 * int(rng.integers(1, 6))]))
        # rows per expert ~ T k / E: reach the streaming (<= 16), 128-row and
        # 256-row tiles
        T = int(rng.choice([1, int(rng.integers(2, 40)), int(rng.integers(40, 400)), int(rng.integers(200, 600))],
                           p=[0.1, 0.3, 0.3, 0.3]))
        route = int(rng.choice(ROUTES))
        rho = float(rng.choice([1.0, 2.5]))
        of = float(rng.choice([0.0, 0.05]))
        max_rows = int(rng.integers(1, T + 1))
        cases.append((f"s{i:02d}_e{E}_k{k}_h{H}_i{I}_t{T}", (E, k, H, I, T, route, rho, of), max_rows))
    return cases


CASES = sweep_cases()


@pytest.mark.parametrize("name,spec,max_rows", CASES)
def test_sweep_matches_oracle(name, spec, max_rows):
    E, k, H, I, T, route, rho, of = spec
    seed = int(name[1:3])
    layer = gen.make_layer(E, H, I, seed=seed)
    x, _ = gen.make_tokens(T, H, seed=seed, outlier_frac=of)
    ids, w = gen.make_routing(T, E, k, route, seed=seed)
    counts = np.bincount(ids[ids >= 0].ravel(), minlength=E)
    note(f"sweep {name}: rows per expert max {counts.max()} min {counts.min()}, passes of {max_rows}")
    od = pkg.MOE_DTYPE_F32 if seed % 2 else pkg.MOE_DTYPE_BF16
    moe = pkg.MoeFp8Prefill(layer, k, routed_scale=rho, out_dtype=od, max_rows=max(T, 1))
    try:
        got = run(moe, x, ids, w)
        assert moe.status() == pkg.MOE_OK
        compare_with_oracle(moe, layer, x, ids, w, rho, got, what=name)
    finally:
        moe.close()
    chunked = pkg.MoeFp8Prefill(layer, k, routed_scale=rho, out_dtype=od, max_rows=max_rows)
    try:
        got2 = run(chunked, x, ids, w)
        assert chunked.status() == pkg.MOE_OK
    finally:
        chunked.close()
    assert np.array_equal(got.view(np.uint8), got2.view(np.uint8)), f"{name}: passes of {max_rows} change bits"
