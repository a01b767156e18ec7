"""The GPU quantizers through the C ABI, bit for bit against the oracle's
table-search encoders, on random BF16 weights with planted edge values
(zero rows and blocks, exact midpoints, tiny and large values, negative
values that round to zero); and a quantized matrix through the product
path against the oracle."""
import numpy as np
import pytest
import torch

import oracle
from oracle import e2m1, e4m3
from oracle.quant import quantize_fp8row, quantize_nvfp4
from fp8_weight_streaming_amd.inputs import to_bf16
from gpu_util import DEV, assert_close, dev_bf16bits, dev_f32, dev_u8, run_fp8, run_nvfp4

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def wq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from fp8_weight_streaming_amd import wq as mod
    return mod


def weights(M, K, seed):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((M, K)) * 0.02 * 10.0 ** rng.uniform(-3, 1, (M, 1))).astype(np.float32)
    w[1] = 0.0                                        # a zero row
    w[2, :32] = 0.0                                   # zero blocks
    w[3, :16] = np.float32(1e-30)                     # blocks whose scale rounds to zero
    w[4, :16] = [6.0, 5.0, 3.5, 2.5, 1.75, 1.25, 0.75, 0.25, -6.0, -5.0, -3.5, -2.5, -1.75, -1.25, -0.75, -0.25]
    if K >= 32:
        w[5, 16:32] = -1e-8                           # negative values that round to zero ...
        w[5, 20] = 1.0                                # ... next to a large one in their block
    return to_bf16(w)


@pytest.mark.parametrize("M,K", [(1, 16), (17, 48), (40, 1040), (300, 5120)])
def test_quantize_fp8row_bit_exact(wq, M, K):
    wb = weights(max(M, 6), K, 10 + M)[:M]
    q = torch.empty((M, K), dtype=torch.uint8, device=DEV)
    r = torch.empty(M, dtype=torch.float32, device=DEV)
    wq.wq_quantize_fp8row(dev_bf16bits(wb), q, r)
    torch.cuda.synchronize()
    qr, rr = quantize_fp8row(wb)
    assert np.array_equal(r.cpu().numpy().view(np.uint32), rr.view(np.uint32)), "row scales"
    assert np.array_equal(q.cpu().numpy(), qr), "codes"


@pytest.mark.parametrize("M,K,g", [(6, 32, 2.0 ** -7), (17, 96, 0.02 / 6), (40, 1056, 1e-3), (300, 5120, 0.5)])
def test_quantize_nvfp4_bit_exact(wq, M, K, g):
    wb = weights(max(M, 6), K, 20 + M)[:M]
    c = torch.empty((M, K // 2), dtype=torch.uint8, device=DEV)
    s = torch.empty((M, K // 16), dtype=torch.uint8, device=DEV)
    wq.wq_quantize_nvfp4(dev_bf16bits(wb), g, c, s)
    torch.cuda.synchronize()
    cr, sr = quantize_nvfp4(wb, np.float32(g))
    assert np.array_equal(s.cpu().numpy(), sr), "scales"
    assert np.array_equal(c.cpu().numpy(), cr), "codes"


def test_quantized_weights_through_the_products(wq):
    # quantize on the GPU, then run both products on the result against the oracle
    from fp8_weight_streaming_amd import inputs
    M, K = 257, 2048
    wb = weights(M, K, 30)
    x = to_bf16(np.random.default_rng(31).standard_normal((8, K)).astype(np.float32))
    q = torch.empty((M, K), dtype=torch.uint8, device=DEV)
    r = torch.empty(M, dtype=torch.float32, device=DEV)
    wq.wq_quantize_fp8row(dev_bf16bits(wb), q, r)
    g = float(np.float32(np.abs((wb.astype(np.uint32) << 16).view(np.float32)).max() / (6 * 448)))
    c = torch.empty((M, K // 2), dtype=torch.uint8, device=DEV)
    s = torch.empty((M, K // 16), dtype=torch.uint8, device=DEV)
    wq.wq_quantize_nvfp4(dev_bf16bits(wb), g, c, s)
    torch.cuda.synchronize()
    d8 = inputs.FP8RowInputs(w=q.cpu().numpy(), row_scale=r.cpu().numpy(), x=x)
    y8 = run_fp8(wq, d8)
    yr, ar = oracle.gemm_fp8row(d8.w, d8.row_scale, x)
    assert_close(y8, yr, ar, "quantized fp8 product")
    d4 = inputs.NVFP4Inputs(codes=c.cpu().numpy(), scales=s.cpu().numpy(), g=g, x=x)
    y4 = run_nvfp4(wq, d4)
    yr, ar = oracle.gemm_nvfp4(d4.codes, d4.scales, g, x)
    assert_close(y4, yr, ar, "quantized nvfp4 product")
