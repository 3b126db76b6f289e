"""gfx950 FP8 MFMA through the library's operand convention (GPU).

Checks that the hardware reads the OCP E4M3 encoding the oracle decodes
("ktransformers #2245", Semantics and scope) and that the library's operand
and result layouts pair K correctly: a one-hot probe over all 254 finite codes
and an exact small-integer product compared with an int64 matmul.
"""
import numpy as np
import pytest
import torch

import fp8_blockwise_routed_amd as pkg
import oracle
from gpu_util import note

pytestmark = pytest.mark.gpu


def test_mfma_decodes_every_finite_code():
    note("mfma probe: one-hot decode of all codes")
    one = 0x38  # 1.0
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    got = np.empty(codes.size, np.float32)
    for start in range(0, codes.size, 16):
        chunk = codes[start:start + 16]
        a = np.zeros((16, 128), np.uint8)
        b = np.zeros((16, 128), np.uint8)
        for i, c in enumerate(chunk):
            a[i, (7 * i + 3) % 128] = c        # one non-zero K position per row
        b[:, :] = one
        d = pkg.moe_fp8_prefill_debug_mfma(a, b)
        for i in range(chunk.size):
            got[start + i] = d[i, 0]
            assert np.all(d[i] == d[i, 0])     # same for every column
    ref = oracle.e4m3_decode(codes)
    # signed zeros: 0x80 * 1.0 summed with +0 products is +0; compare values
    assert np.array_equal(got, ref), np.nonzero(got != ref)


def test_mfma_small_integer_product_is_exact():
    note("mfma probe: integer product")
    rng = np.random.default_rng(0)
    av = rng.integers(-8, 9, (16, 128)).astype(np.float32)
    bv = rng.integers(-8, 9, (16, 128)).astype(np.float32)
    enc = lambda v: torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    d = pkg.moe_fp8_prefill_debug_mfma(enc(av), enc(bv))
    ref = av.astype(np.int64) @ bv.astype(np.int64).T
    assert np.array_equal(d.astype(np.int64), ref)


def test_mfma_rows_and_columns_land_in_place():
    note("mfma probe: row/column placement")
    a = np.zeros((16, 128), np.uint8)
    b = np.zeros((16, 128), np.uint8)
    enc = lambda v: int(torch.tensor([float(v)]).to(torch.float8_e4m3fn).view(torch.uint8)[0])
    for i in range(16):
        a[i, i] = enc(i + 1)            # row i uses K=i with value i+1
        b[i, :16] = 0
    for n in range(16):
        for kk in range(16):
            b[n, kk] = enc(1.0 if kk == (n % 16) or kk < 0 else 0.0)
    # d[i][n] = (i+1) * [n == i]
    d = pkg.moe_fp8_prefill_debug_mfma(a, b)
    assert np.array_equal(d, np.diag(np.arange(1, 17, dtype=np.float32)))
