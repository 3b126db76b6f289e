"""moe_fp8_prefill_run_static (the entry point that allocates nothing, its
per-pass workspace in the library's static device array) against
moe_fp8_prefill_run on the same inputs (GPU).

The two share every kernel, and a row's bits do not depend on how the rows
are split into passes, so the outputs must be equal bit for bit: on two calls
in a row, the second with fewer rows; on a layer whose rows need several
passes of the static array; and the device's free memory must not change
across static calls.
"""
import numpy as np
import pytest
import torch

import fp8_blockwise_routed_amd as pkg
import gen
from gpu_util import dev, dev_bf16, note

pytestmark = pytest.mark.gpu

# (name, E, k, H, I, T first call, T second call, route, rho)
CASES = [
    ("tiny", 8, 2, 256, 128, 64, 17, gen.ROUTE_SOFTMAX, 1.0),
    # E=16 experts of the GLM shape: ~220 KB of workspace per row, so the
    # 700-row call runs in three passes of the 64 MiB array
    ("glm_shape", 16, 8, 6144, 2048, 700, 50, gen.ROUTE_SIGMOID_NORMAL, 2.5),
]


def call(fn, moe, x, ids, w, out):
    rc = fn(moe.handle, x, ids, w, x.shape[0], out)
    assert rc == pkg.MOE_OK, pkg.moe_fp8_prefill_strerror(rc)
    return out


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
@pytest.mark.parametrize("out_dtype", [pkg.MOE_DTYPE_BF16, pkg.MOE_DTYPE_F32])
def test_run_static_equals_run(case, out_dtype):
    name, E, k, H, I, T1, T2, route, rho = case
    layer = gen.make_layer(E, H, I, seed=2)
    x, _ = gen.make_tokens(T1, H, seed=2, outlier_frac=0.01)
    ids, w = gen.make_routing(T1, E, k, route, seed=2)
    dtype = torch.float32 if out_dtype == pkg.MOE_DTYPE_F32 else torch.bfloat16
    moe = pkg.MoeFp8Prefill(layer, k, routed_scale=rho, out_dtype=out_dtype)
    try:
        xd, idd, wd = dev_bf16(x), dev(ids), dev(w)
        for T in (T1, T2):
            note(f"run_static {name} out_dtype={out_dtype} T={T}")
            ref = torch.empty((T, H), dtype=dtype, device="cuda")
            got = torch.full((T, H), 7, dtype=dtype, device="cuda")
            call(pkg.moe_fp8_prefill_run, moe, xd[:T], idd[:T], wd[:T], ref)
            torch.cuda.synchronize()
            free0 = torch.cuda.mem_get_info()[0]
            call(pkg.moe_fp8_prefill_run_static, moe, xd[:T], idd[:T], wd[:T], got)
            torch.cuda.synchronize()
            assert torch.cuda.mem_get_info()[0] == free0, "run_static changed the device's free memory"
            assert moe.status() == pkg.MOE_OK
            assert torch.equal(got.view(torch.int16) if dtype == torch.bfloat16 else got.view(torch.int32),
                               ref.view(torch.int16) if dtype == torch.bfloat16 else ref.view(torch.int32)), \
                f"{name} T={T}: run_static differs from run"
    finally:
        moe.close()


def test_run_static_rejects_bad_arguments():
    layer = gen.make_layer(8, 256, 128, seed=2)
    moe = pkg.MoeFp8Prefill(layer, 2)
    try:
        out = torch.empty((1, 256), dtype=torch.bfloat16, device="cuda")
        assert pkg.moe_fp8_prefill_run_static(moe.handle, None, None, None, 1, out) == pkg.MOE_ERR_INVALID_ARG
        assert pkg.moe_fp8_prefill_run_static(moe.handle, None, None, None, 0, None) == pkg.MOE_OK
    finally:
        moe.close()
    assert pkg.moe_fp8_prefill_run_static(0, None, None, None, 1, None) == pkg.MOE_ERR_INVALID_ARG
