"""Tiled NVFP4 on the GPU: the conversion kernels match the layout's numpy
statement byte for byte and invert exactly; the tiled product matches the
oracle, and the plain product bit for bit when both use the same K split."""
import numpy as np
import pytest
import torch

import oracle
from fp8_weight_streaming_amd import inputs
from gpu_util import DEV, assert_close, dev_bf16bits, dev_u8, run_nvfp4, workspace
from tiled_ref import tile_ref

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def wq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from fp8_weight_streaming_amd import wq as mod
    return mod


def to_tiled(wq, d):
    t = torch.empty(wq.wq_nvfp4_tiled_bytes(d.M, d.K), dtype=torch.uint8, device=DEV)
    wq.wq_nvfp4_tile(dev_u8(d.codes), dev_u8(d.scales), t)
    return t


def run_tiled(wq, d, N, x=None):
    x = d.x if x is None else x
    t = to_tiled(wq, d)
    y = torch.full((N, d.M), float("nan"), dtype=torch.float32, device=DEV)
    ws = workspace(wq.wq_gemm_workspace_bytes(wq.WQ_FMT_NVFP4_TILED, d.M, d.K, N))
    wq.wq_gemm_nvfp4_tiled(t, d.g, dev_bf16bits(x[:N]), y, d.M, d.K, ws)
    torch.cuda.synchronize()
    return y.cpu().numpy()


SHAPES = [(1, 32), (16, 256), (17, 96), (33, 160), (100, 544), (64, 1024), (250, 4224), (48, 8736), (40, 17440),
          (7168, 5120)]


@pytest.mark.parametrize("M,K", SHAPES)
def test_tile_matches_layout_and_inverts(wq, M, K):
    d = inputs.nvfp4_inputs(M, K, 1, seed=300 + M + K)
    t = to_tiled(wq, d)
    torch.cuda.synchronize()
    assert np.array_equal(t.cpu().numpy(), tile_ref(d.codes, d.scales)), "tiled bytes differ"
    c = torch.zeros((M, K // 2), dtype=torch.uint8, device=DEV)
    s = torch.zeros((M, K // 16), dtype=torch.uint8, device=DEV)
    wq.wq_nvfp4_untile(t, c, s)
    torch.cuda.synchronize()
    assert np.array_equal(c.cpu().numpy(), d.codes) and np.array_equal(s.cpu().numpy(), d.scales)


@pytest.mark.parametrize("M,K", SHAPES[:-1])
def test_tiled_gemm_all_n(wq, M, K):
    d = inputs.nvfp4_inputs(M, K, 8, seed=400 + M + K, g=0.02)
    same = wq.wq_gemm_split(wq.WQ_FMT_NVFP4, M, K) == wq.wq_gemm_split(wq.WQ_FMT_NVFP4_TILED, M, K)
    print("M=%d K=%d split plain=%s tiled=%s" % (M, K, wq.wq_gemm_split(0, M, K), wq.wq_gemm_split(2, M, K)),
          flush=True)
    for N in range(1, 9):
        y = run_tiled(wq, d, N)
        yr, ar = oracle.gemm_nvfp4(d.codes, d.scales, d.g, d.x[:N])
        assert_close(y, yr, ar, "tiled M=%d K=%d N=%d" % (M, K, N))
        if same:
            yp = run_nvfp4(wq, d, N)
            assert np.array_equal(yp.view(np.uint32), y.view(np.uint32)), "tiled vs plain bits N=%d" % N


def test_tiled_column_invariance(wq):
    d = inputs.nvfp4_inputs(96, 17408, 8, seed=9, g=0.02)
    y8 = run_tiled(wq, d, 8)
    for N in (1, 3, 5, 7):
        assert np.array_equal(run_tiled(wq, d, N).view(np.uint32), y8[:N].view(np.uint32))
    for j in (0, 5, 7):
        assert np.array_equal(run_tiled(wq, d, 1, x=d.x[j:j + 1])[0].view(np.uint32), y8[j].view(np.uint32))


@pytest.mark.parametrize("N", [2, 8])
def test_tiled_verify_pass_dense_layer(wq, N):
    specs = inputs.VERIFY_LAYER
    mats, host, keep = [], [], []
    for i, s in enumerate(specs):
        d = inputs.nvfp4_inputs(s.M, s.K, N, seed=950 + i, g=0.02)
        t = to_tiled(wq, d)
        y = torch.full((N, s.M), float("nan"), dtype=torch.float32, device=DEV)
        x = dev_bf16bits(d.x)
        mats.append(wq.Matrix(wq.WQ_FMT_NVFP4_TILED, s.M, s.K, t, None, x, y, d.g))
        host.append(d)
        keep.append((t, x))
    ws = workspace(wq.wq_verify_workspace_bytes(mats, N))
    wq.wq_verify_pass(mats, N, ws)
    torch.cuda.synchronize()
    rng = np.random.default_rng(77 + N)
    for m, d in zip(mats, host):
        rows = np.unique(np.concatenate([rng.integers(0, m.M, 500), [0, m.M - 1]]))
        yr, ar = oracle.gemm_nvfp4(d.codes, d.scales, d.g, d.x, rows=rows)
        assert_close(m.y.cpu().numpy()[:, rows], yr, ar, "tiled pass M=%d K=%d N=%d" % (m.M, m.K, N))


def test_tiled_verify_pass_column_invariance(wq):
    # Long rows are staged in one K chunk when the N columns fit in LDS
    # (N <= 4 here) and in two otherwise; both must give the same bits,
    # including a ragged last summation chunk (K = 17440).
    specs = [(96, 17408), (40, 17440), (33, 8736), (17, 544)]
    host = [inputs.nvfp4_inputs(M, K, 8, seed=1200 + i, g=0.02) for i, (M, K) in enumerate(specs)]
    tiled = [to_tiled(wq, d) for d in host]
    xs = [dev_bf16bits(d.x) for d in host]
    outs = {}
    for N in range(1, 9):
        mats = []
        for d, t, x in zip(host, tiled, xs):
            y = torch.full((N, d.M), float("nan"), dtype=torch.float32, device=DEV)
            mats.append(wq.Matrix(wq.WQ_FMT_NVFP4_TILED, d.M, d.K, t, None, x[:N].contiguous(), y, d.g))
        ws = workspace(wq.wq_verify_workspace_bytes(mats, N))
        print("column invariance N=%d workspace=%d" % (N, 0 if ws is None else ws.numel()), flush=True)
        wq.wq_verify_pass(mats, N, ws)
        torch.cuda.synchronize()
        outs[N] = [m.y.cpu().numpy() for m in mats]
    for i, d in enumerate(host):
        yr, ar = oracle.gemm_nvfp4(d.codes, d.scales, d.g, d.x)
        assert_close(outs[8][i], yr, ar, "pass M=%d K=%d N=8" % (d.M, d.K))
        for N in range(1, 8):
            assert np.array_equal(outs[N][i].view(np.uint32), outs[8][i][:N].view(np.uint32)), \
                "M=%d K=%d: N=%d differs from N=8" % (d.M, d.K, N)
