"""The largest matrices the tiled layouts address: just under 2**32 bytes of
tiled weights (the kernels compute weight offsets in 32 bits).  Built on the
device from hashed rows, chunk by chunk; the oracle checks sampled rows (the
first and last 16, the 16 of the tile whose blocks cross 2**31 bytes, and
32 others), and every output must be written (all outputs start as NaN and
every input is finite)."""
import numpy as np
import pytest
import torch

import oracle
from fp8_weight_streaming_amd import inputs
from gpu_util import DEV, assert_close, dev_bf16bits, workspace

pytestmark = pytest.mark.gpu

CHUNK = 65536  # rows generated and uploaded at a time
N = 8


@pytest.fixture(scope="module")
def wq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from fp8_weight_streaming_amd import wq as mod
    return mod


def sample_rows(M, tile_bytes, seed):
    t_cross = (1 << 31) // tile_bytes  # first tile with blocks past 2**31 bytes
    rng = np.random.default_rng(seed)
    rows = np.concatenate([np.arange(16), np.arange(M - 16, M), np.arange(16 * t_cross, 16 * t_cross + 16),
                           rng.integers(0, M, 32)])
    return np.unique(rows)


def check_all_written(y, what):
    assert bool(torch.isfinite(y).all()), "%s: outputs left unwritten or not finite" % what


def test_largest_tiled_nvfp4(wq):
    M, K, seed = 438600, 17408, 3100
    nbytes = wq.wq_nvfp4_tiled_bytes(M, K)
    assert nbytes < (1 << 32) and nbytes + 68 * 2304 >= (1 << 32), nbytes  # one more tile would not fit
    codes = torch.empty((M, K // 2), dtype=torch.uint8, device=DEV)
    scales = torch.empty((M, K // 16), dtype=torch.uint8, device=DEV)
    for r0 in range(0, M, CHUNK):
        c, s = inputs.hashed_nvfp4_rows(np.arange(r0, min(r0 + CHUNK, M)), K, seed)
        codes[r0:r0 + len(c)].copy_(torch.from_numpy(c))
        scales[r0:r0 + len(s)].copy_(torch.from_numpy(s))
    t = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    wq.wq_nvfp4_tile(codes, scales, t)
    torch.cuda.synchronize()
    del codes, scales
    g = 0.02
    x = inputs.nvfp4_inputs(1, K, N, seed=seed).x
    xd = dev_bf16bits(x)
    rows = sample_rows(M, 68 * 2304, seed)
    c, s = inputs.hashed_nvfp4_rows(rows, K, seed)
    yr, ar = oracle.gemm_nvfp4(c, s, np.float32(g), x)
    # the single product (K in two chunks, then the reduction launch)
    y = torch.full((N, M), float("nan"), dtype=torch.float32, device=DEV)
    ws = workspace(wq.wq_gemm_workspace_bytes(wq.WQ_FMT_NVFP4_TILED, M, K, N))
    print("largest nvfp4 %dx%d single product" % (M, K), flush=True)
    wq.wq_gemm_nvfp4_tiled(t, g, xd, y, M, K, ws)
    torch.cuda.synchronize()
    check_all_written(y, "nvfp4 single product")
    assert_close(y[:, torch.from_numpy(rows).to(DEV)].cpu().numpy(), yr, ar, "nvfp4 single product")
    # a one-matrix verify pass (K in blocks of three chunks kept in LDS)
    y2 = torch.full((N, M), float("nan"), dtype=torch.float32, device=DEV)
    mats = [wq.Matrix(wq.WQ_FMT_NVFP4_TILED, M, K, t, None, xd, y2, g)]
    ws2 = workspace(wq.wq_verify_workspace_bytes(mats, N))
    print("largest nvfp4 %dx%d verify pass" % (M, K), flush=True)
    wq.wq_verify_pass(mats, N, ws2)
    torch.cuda.synchronize()
    check_all_written(y2, "nvfp4 verify pass")
    assert_close(y2[:, torch.from_numpy(rows).to(DEV)].cpu().numpy(), yr, ar, "nvfp4 verify pass")


def test_largest_tiled_fp8(wq):
    M, K, seed = 838840, 5120, 3200
    nbytes = wq.wq_fp8_tiled_bytes(M, K)
    assert nbytes < (1 << 32) and nbytes + 40 * 2048 >= (1 << 32), nbytes
    w = torch.empty((M, K), dtype=torch.uint8, device=DEV)
    rs = torch.empty(M, dtype=torch.float32, device=DEV)
    for r0 in range(0, M, CHUNK):
        wc, rc = inputs.hashed_fp8_rows(np.arange(r0, min(r0 + CHUNK, M)), K, seed)
        w[r0:r0 + len(wc)].copy_(torch.from_numpy(wc))
        rs[r0:r0 + len(rc)].copy_(torch.from_numpy(rc))
    t = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    wq.wq_fp8_tile(w, t)
    torch.cuda.synchronize()
    del w
    x = inputs.fp8row_inputs(1, K, N, seed=seed).x
    xd = dev_bf16bits(x)
    rows = sample_rows(M, 40 * 2048, seed)
    wc, rc = inputs.hashed_fp8_rows(rows, K, seed)
    yr, ar = oracle.gemm_fp8row(wc, rc, x)
    y = torch.full((N, M), float("nan"), dtype=torch.float32, device=DEV)
    ws = workspace(wq.wq_gemm_workspace_bytes(wq.WQ_FMT_FP8ROW_TILED, M, K, N))
    print("largest fp8 %dx%d single product" % (M, K), flush=True)
    wq.wq_gemm_fp8row_tiled(t, rs, xd, y, M, K, ws)
    torch.cuda.synchronize()
    check_all_written(y, "fp8 single product")
    assert_close(y[:, torch.from_numpy(rows).to(DEV)].cpu().numpy(), yr, ar, "fp8 single product")
    # the same matrix as a one-matrix verify pass: same K split, same bits
    y2 = torch.full((N, M), float("nan"), dtype=torch.float32, device=DEV)
    mats = [wq.Matrix(wq.WQ_FMT_FP8ROW_TILED, M, K, t, rs, xd, y2)]
    ws2 = workspace(wq.wq_verify_workspace_bytes(mats, N))
    print("largest fp8 %dx%d verify pass" % (M, K), flush=True)
    wq.wq_verify_pass(mats, N, ws2)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int32), y2.view(torch.int32)), "fp8 verify pass differs from the single product"
