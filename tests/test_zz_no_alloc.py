"""wq_gemm_nvfp4_tiled_noalloc (split-K scratch in the library's static
device buffer) against wq_gemm_nvfp4_tiled with a workspace: the same bits,
on two calls in a row, the second with a smaller input; and a shape whose
scratch would not fit is refused with nothing launched."""
import numpy as np
import pytest
import torch

from fp8_weight_streaming_amd import inputs
from gpu_util import DEV, dev_bf16bits, dev_u8, workspace

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def wq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from fp8_weight_streaming_amd import wq as mod
    return mod


def tiled_of(wq, d):
    t = torch.empty(wq.wq_nvfp4_tiled_bytes(d.M, d.K), dtype=torch.uint8, device=DEV)
    wq.wq_nvfp4_tile(dev_u8(d.codes), dev_u8(d.scales), t)
    return t


def test_noalloc_matches_workspace_call_twice(wq):
    # a product with many tiles per CU (the chunked stream kernel, its chunk
    # sums in the scratch for a reduction, its outputs held in LDS), the
    # down-projection shape at N = 8 (split across workgroups), then a
    # smaller split shape at N = 3 with a ragged last tile and chunk
    cases = [(36001, 10240, 8, 2100), (5120, 17408, 8, 2101), (1000, 8736, 3, 2102)]
    for M, K, N, seed in cases:
        need = wq.wq_gemm_workspace_bytes(wq.WQ_FMT_NVFP4_TILED, M, K, N)
        print("noalloc case M=%d K=%d N=%d scratch %d bytes" % (M, K, N, need), flush=True)
        assert 0 < need <= wq.NOALLOC_SCRATCH_BYTES, "the case must use the scratch buffer"
        d = inputs.nvfp4_inputs(M, K, N, seed=seed, g=0.02)
        t, x = tiled_of(wq, d), dev_bf16bits(d.x)
        y_ref = torch.full((N, M), float("nan"), dtype=torch.float32, device=DEV)
        wq.wq_gemm_nvfp4_tiled(t, d.g, x, y_ref, M, K, workspace(need))
        y = torch.full((N, M), float("nan"), dtype=torch.float32, device=DEV)
        wq.wq_gemm_nvfp4_tiled_noalloc(t, d.g, x, y, M, K)
        torch.cuda.synchronize()
        a, b = y_ref.cpu().numpy(), y.cpu().numpy()
        assert not np.isnan(a).any()
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), "M=%d K=%d N=%d: bits differ" % (M, K, N)


def test_noalloc_refuses_shapes_past_its_scratch(wq):
    M, K, N = 151936, 17408, 8
    need = wq.wq_gemm_workspace_bytes(wq.WQ_FMT_NVFP4_TILED, M, K, N)
    assert need > wq.NOALLOC_SCRATCH_BYTES
    y = torch.zeros((N, 16), dtype=torch.float32, device=DEV)
    fake = y  # never read: the call is refused before any launch
    with pytest.raises(wq.WQError) as e:
        wq.wq_gemm_nvfp4_tiled_noalloc(fake, 1.0, fake, y, M, K, N=N)
    assert e.value.status == 7
    torch.cuda.synchronize()
    assert (y.cpu().numpy() == 0).all()
