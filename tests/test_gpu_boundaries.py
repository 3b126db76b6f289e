"""Experts whose row counts sit on the GEMM variants' limits (GPU).

One layer, top-2 routing built so that expert e receives exactly ROWS[e]
rows: none, one, and both sides of the 16-row streaming limit, the 128-row
tile and the 256-row tile (one tile, one full tile plus a one-row tile, two
full tiles plus one row).  The output is compared with the oracle (staged
checks and the plain per-row bound), the plan's counts with ROWS, and runs
in passes of fewer rows must give the same bits.
"""
import numpy as np
import pytest

import fp8_blockwise_routed_amd as pkg
import gen
from gpu_util import compare_with_oracle, note, run

pytestmark = pytest.mark.gpu

ROWS = [0, 1, 15, 16, 17, 64, 127, 128, 129, 255, 256, 257, 384, 512, 513]
H, I = 512, 1024


def boundary_routing(seed=7):
    """Top-2 ids and weights with exactly ROWS[e] slots on expert e."""
    rng = np.random.default_rng(seed)
    slots = np.repeat(np.arange(len(ROWS), dtype=np.int32), ROWS)  # sorted by expert
    half = slots.size // 2
    assert slots.size % 2 == 0 and max(ROWS) <= half
    # slot i and slot i + half are different experts (no expert fills half)
    ids = np.stack([slots[:half], slots[half:]], axis=1)
    ids = ids[rng.permutation(half)]
    swap = rng.random(half) < 0.5
    ids[swap] = ids[swap][:, ::-1]
    w = rng.random((half, 2)).astype(np.float32) + 0.05
    w /= w.sum(axis=1, keepdims=True)
    return np.ascontiguousarray(ids), w


@pytest.mark.parametrize("out_dtype", [pkg.MOE_DTYPE_BF16, pkg.MOE_DTYPE_F32])
def test_tile_limits(out_dtype):
    ids, w = boundary_routing()
    T = ids.shape[0]
    assert np.array_equal(np.bincount(ids.ravel(), minlength=len(ROWS)), ROWS)
    layer = gen.make_layer(len(ROWS), H, I, seed=11)
    x, _ = gen.make_tokens(T, H, seed=11, outlier_frac=0.01)
    note(f"tile limits: T={T} rows per expert {ROWS} out_dtype={out_dtype}")
    moe = pkg.MoeFp8Prefill(layer, 2, routed_scale=2.5, out_dtype=out_dtype, max_rows=T)
    try:
        got = run(moe, x, ids, w)
        assert moe.status() == pkg.MOE_OK
        counts = pkg.moe_fp8_prefill_debug_plan(moe.handle, len(ROWS), T * 2)[0]
        assert np.array_equal(np.asarray(counts)[: len(ROWS)], ROWS)
        compare_with_oracle(moe, layer, x, ids, w, 2.5, got, what=f"tile limits {out_dtype}")
    finally:
        moe.close()
    for max_rows in (97, 300):
        chunked = pkg.MoeFp8Prefill(layer, 2, routed_scale=2.5, out_dtype=out_dtype, max_rows=max_rows)
        try:
            got2 = run(chunked, x, ids, w)
            assert chunked.status() == pkg.MOE_OK
        finally:
            chunked.close()
        assert np.array_equal(got.view(np.uint8), got2.view(np.uint8)), f"passes of {max_rows} change bits"
