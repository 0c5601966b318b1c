"""GPU test of the matrix-core rate probe (a measurement aid used by the benchmark).

With every operand element equal to c, each 32x32x16 product adds 16 c^2 to
every accumulator element (a binary32 32x32x2 product 2 c^2, an E4M3 32x32x64
product 64 c^2), so after mfma_per_wave / 16 products per chain a lane's 16
chains x 16 registers sum to 256 * 16 * c^2 * (mfma_per_wave / 16) (256 * 2 *
... for binary32, 256 * 64 * ... for E4M3): exact in FP32 for the small counts
used here.
"""
import pytest
import torch

import layout_algebra_amd as la

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16, torch.float32, torch.float8_e4m3fn])
@pytest.mark.parametrize("c", [1.0, 2.0, -0.5])
def test_probe_accumulates_exact_products(dtype, c):
    wg, n = 8, 64
    ops = torch.full((4096,), c, dtype=dtype).to(DEV)
    sink = torch.full((wg * 256,), float("nan"), dtype=torch.float32, device=DEV)
    la.la_probe_mfma(ops, sink, wg, n)
    torch.cuda.synchronize()
    depth = {torch.float32: 2.0, torch.float8_e4m3fn: 64.0}.get(dtype, 16.0)
    expect = 256.0 * depth * c * c * (n // 16)
    assert torch.all(sink.cpu() == expect), sink.cpu()[:8]


def test_probe_rejects_bad_arguments():
    ops = torch.ones(4096, dtype=torch.bfloat16, device=DEV)
    sink = torch.empty(256, dtype=torch.float32, device=DEV)
    with pytest.raises(la.GemmError):
        la.la_probe_mfma(ops, sink, 1, 24)           # not a multiple of 16
    with pytest.raises(ValueError):
        la.la_probe_mfma(ops, sink, 2, 16)           # sink too small for 2 workgroups
