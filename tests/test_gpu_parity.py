"""Parity of the HIP path with the CPU oracle, through the C ABI.

Every case compares each output element with the oracle's FP64 value under
|y_gpu - y| <= 1e-3 * sum_k |w x| and requires NaN exactly where the oracle
has NaN.  Shapes span several 16-row tiles, ragged M and K tails, every N
from 1 to 8, split and unsplit K, and the five workloads at full size.
"""
import numpy as np
import pytest
import torch

import oracle
from fp8_weight_streaming_amd import inputs
from gpu_util import (DEV, assert_close, check_fp8, check_nvfp4, dev_bf16bits, dev_f32, dev_u8, run_fp8,
                      run_nvfp4, workspace)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def wq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from fp8_weight_streaming_amd import wq as mod
    return mod


NV_SHAPES = [(1, 32), (16, 128), (17, 96), (33, 160), (100, 544), (64, 1024), (250, 4224), (48, 8736),
             (40, 17440)]


@pytest.mark.parametrize("M,K", NV_SHAPES)
def test_nvfp4_shapes_all_n(wq, M, K):
    d = inputs.nvfp4_inputs(M, K, 8, seed=100 + M + K, g=0.02)
    print("nvfp4 M=%d K=%d split=%s" % (M, K, wq.wq_gemm_split(wq.WQ_FMT_NVFP4, M, K)), flush=True)
    for N in range(1, 9):
        check_nvfp4(wq, d, N, what="nvfp4 M=%d K=%d N=%d" % (M, K, N))


FP8_SHAPES = [(1, 16), (5, 48), (16, 64), (17, 80), (40, 1040), (300, 5120), (33, 8720)]


@pytest.mark.parametrize("M,K", FP8_SHAPES)
def test_fp8row_shapes_all_n(wq, M, K):
    d = inputs.fp8row_inputs(M, K, 8, seed=200 + M + K)
    print("fp8row M=%d K=%d split=%s" % (M, K, wq.wq_gemm_split(wq.WQ_FMT_FP8ROW, M, K)), flush=True)
    for N in range(1, 9):
        check_fp8(wq, d, N, what="fp8row M=%d K=%d N=%d" % (M, K, N))


@pytest.mark.parametrize("index", [0, 1, 2])
def test_workload_nvfp4_full(wq, index):
    wl = inputs.workload(index)
    d = inputs.workload_inputs(wl, 0)
    print("workload %d: %s, split=%s" % (index, wl.name, wq.wq_gemm_split(wq.WQ_FMT_NVFP4, d.M, d.K)), flush=True)
    check_nvfp4(wq, d, wl.N, what=wl.name)


def test_workload_fp8_head_sampled(wq):
    wl = inputs.workload(4)
    d = inputs.workload_inputs(wl, 0)
    rng = np.random.default_rng(4)
    rows = np.unique(np.concatenate([rng.integers(0, d.M, 3000), [0, 1, 15, 16, d.M - 1]]))
    print("workload 4: %s, split=%s" % (wl.name, wq.wq_gemm_split(wq.WQ_FMT_FP8ROW, d.M, d.K)), flush=True)
    check_fp8(wq, d, wl.N, rows=rows, what=wl.name)


def test_column_invariance_and_repeat(wq):
    for fmt in ("nvfp4", "fp8"):
        if fmt == "nvfp4":
            d = inputs.nvfp4_inputs(130, 17408, 8, seed=7, g=0.02)
            run = run_nvfp4
        else:
            d = inputs.fp8row_inputs(130, 5120, 8, seed=7)
            run = run_fp8
        y8 = run(wq, d, 8)
        again = run(wq, d, 8)
        assert np.array_equal(y8.view(np.uint32), again.view(np.uint32)), fmt + ": repeat differs"
        for N in range(1, 8):
            yN = run(wq, d, N)
            assert np.array_equal(yN.view(np.uint32), y8[:N].view(np.uint32)), "%s: N=%d differs" % (fmt, N)
        for j in range(8):
            yj = run(wq, d, 1, x=d.x[j:j + 1])
            assert np.array_equal(yj[0].view(np.uint32), y8[j].view(np.uint32)), "%s: column %d alone" % (fmt, j)


def test_edge_values_nvfp4(wq):
    M, K = 48, 256
    d = inputs.nvfp4_inputs(M, K, 8, seed=3, g=1.0)
    d.scales[0, :] = 0x7F           # NaN scales: row 0 all NaN
    d.scales[1, 3] = 0xFF           # one NaN block in row 1
    d.scales[2, :] = 0x00           # zero scales
    d.scales[3, :] = 0x7E           # 448
    d.codes[3, :] = 0x77            # +6 everywhere: 6 * 448 = 2688 per weight
    d.scales[4, :] = 0x01           # smallest subnormal scale
    d.codes[5, :] = 0x88            # -0 codes
    d.x[6, :] = 0                   # one zero column
    d.x[7, :] = 0x7180              # 2^100 in one column (large, no FP32 overflow)
    d.x[7, ::2] = 0x0D80            # and 2^-100 in half of it
    y = run_nvfp4(wq, d, 8)
    yr, ar = oracle.gemm_nvfp4(d.codes, d.scales, d.g, d.x)
    assert_close(y, yr, ar, "edge nvfp4")
    assert np.all(np.isnan(y[:, 0])) and np.isnan(y[0, 1]) and not np.isnan(y[0, 2])
    assert np.all(y[6, 2:] == 0)


def test_edge_values_fp8(wq):
    M, K = 40, 128
    d = inputs.fp8row_inputs(M, K, 4, seed=5)
    d.w[0, 5] = 0x7F                # NaN weight
    d.row_scale[1] = 0.0            # zero row
    d.w[2, :] = 0x7E                # 448
    d.row_scale[2] = 1.0
    y = run_fp8(wq, d, 4)
    yr, ar = oracle.gemm_fp8row(d.w, d.row_scale, d.x)
    assert_close(y, yr, ar, "edge fp8")
    assert np.all(np.isnan(y[:, 0])) and np.all(y[:, 1] == 0)


def test_split_workspace_reuse(wq):
    # a split-K shape, then a different split-K shape on the same workspace,
    # then the first again: counters must be back at zero after every call
    a = inputs.nvfp4_inputs(64, 8192, 4, seed=1, g=0.02)
    b = inputs.nvfp4_inputs(200, 4096, 4, seed=2, g=0.02)
    na = wq.wq_gemm_workspace_bytes(wq.WQ_FMT_NVFP4, a.M, a.K, 4)
    nb = wq.wq_gemm_workspace_bytes(wq.WQ_FMT_NVFP4, b.M, b.K, 4)
    assert na > 0 and nb > 0
    ws = workspace(max(na, nb))
    outs = []
    for d in (a, b, a):
        y = torch.empty((4, d.M), dtype=torch.float32, device=DEV)
        wq.wq_gemm_nvfp4(dev_u8(d.codes), dev_u8(d.scales), d.g, dev_bf16bits(d.x), y, ws)
        torch.cuda.synchronize()
        outs.append(y.cpu().numpy())
        yr, ar = oracle.gemm_nvfp4(d.codes, d.scales, d.g, d.x)
        assert_close(outs[-1], yr, ar, "reuse M=%d" % d.M)
    assert np.array_equal(outs[0].view(np.uint32), outs[2].view(np.uint32))
    assert int(ws.sum().item()) >= 0


def _pass_mats(wq, specs, N, seed0):
    mats, host = [], []
    for i, (fmt, M, K) in enumerate(specs):
        if fmt == "nvfp4":
            d = inputs.nvfp4_inputs(M, K, N, seed=seed0 + i, g=0.02)
            y = torch.full((N, M), float("nan"), dtype=torch.float32, device=DEV)
            mats.append(wq.Matrix(wq.WQ_FMT_NVFP4, M, K, dev_u8(d.codes), dev_u8(d.scales), dev_bf16bits(d.x), y,
                                  d.g))
        else:
            d = inputs.fp8row_inputs(M, K, N, seed=seed0 + i)
            y = torch.full((N, M), float("nan"), dtype=torch.float32, device=DEV)
            mats.append(wq.Matrix(wq.WQ_FMT_FP8ROW, M, K, dev_u8(d.w), dev_f32(d.row_scale), dev_bf16bits(d.x), y))
        host.append((fmt, d))
    return mats, host


@pytest.mark.parametrize("N", [1, 3, 8])
def test_verify_pass_mixed(wq, N):
    specs = [("nvfp4", 100, 544), ("fp8", 70, 1040), ("nvfp4", 33, 17440), ("nvfp4", 512, 5120),
             ("fp8", 16, 64), ("nvfp4", 1, 32), ("nvfp4", 40, 8736)]
    mats, host = _pass_mats(wq, specs, N, 500)
    ws = workspace(wq.wq_verify_workspace_bytes(mats, N))
    wq.wq_verify_pass(mats, N, ws)
    torch.cuda.synchronize()
    for m, (fmt, d) in zip(mats, host):
        y = m.y.cpu().numpy()
        if fmt == "nvfp4":
            yr, ar = oracle.gemm_nvfp4(d.codes, d.scales, d.g, d.x)
        else:
            yr, ar = oracle.gemm_fp8row(d.w, d.row_scale, d.x)
        assert_close(y, yr, ar, "pass %s M=%d K=%d N=%d" % (fmt, m.M, m.K, N))
        # same split -> same bits as the single-matrix call
        if wq.wq_gemm_split(m.fmt, m.M, m.K) == wq.wq_gemm_split(m.fmt, m.M, m.K, True):
            ys = run_nvfp4(wq, d, N) if fmt == "nvfp4" else run_fp8(wq, d, N)
            assert np.array_equal(ys.view(np.uint32), y.view(np.uint32)), "pass vs gemm bits M=%d" % m.M


@pytest.mark.parametrize("N", [2, 4, 8])
def test_verify_pass_dense_layers(wq, N):
    # the dense verify-pass shapes (two layers), sampled rows against the oracle
    specs = [("nvfp4", s.M, s.K) for _ in range(2) for s in inputs.VERIFY_LAYER]
    mats, host = _pass_mats(wq, specs, N, 900)
    ws = workspace(wq.wq_verify_workspace_bytes(mats, N))
    wq.wq_verify_pass(mats, N, ws)
    torch.cuda.synchronize()
    rng = np.random.default_rng(N)
    for m, (fmt, d) in zip(mats, host):
        rows = np.unique(np.concatenate([rng.integers(0, m.M, 400), [0, 15, 16, m.M - 1]]))
        yr, ar = oracle.gemm_nvfp4(d.codes, d.scales, d.g, d.x, rows=rows)
        assert_close(m.y.cpu().numpy()[:, rows], yr, ar, "dense pass M=%d K=%d N=%d" % (m.M, m.K, N))
