"""The verify pass with its NVFP4 steps on the vector ALUs
(wq_verify_launch_valu), the comparison that prices the matrix-core step:
against the oracle, and column n the same bits for every N."""
import numpy as np
import pytest
import torch

import oracle
from fp8_weight_streaming_amd import inputs
from gpu_util import DEV, assert_close, dev_bf16bits, dev_u8, workspace

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


@pytest.mark.parametrize("N", [1, 2, 8])
def test_valu_dense_layer(wq, N):
    mats, host, keep = [], [], []
    for i, s in enumerate(inputs.VERIFY_LAYER):
        d = inputs.nvfp4_inputs(s.M, s.K, N, seed=2200 + i, g=0.02)
        t, x = to_tiled(wq, d), dev_bf16bits(d.x)
        y = torch.full((N, s.M), float("nan"), dtype=torch.float32, device=DEV)
        mats.append(wq.Matrix(wq.WQ_FMT_NVFP4_TILED, s.M, s.K, t, None, x, y, d.g))
        host.append(d)
        keep.append((t, x))
    ws = workspace(wq.wq_verify_workspace_bytes(mats, N))
    plan = wq.wq_verify_prepare(mats, N, ws)
    print("valu dense layer N=%d" % N, flush=True)
    wq.wq_verify_launch_valu(plan)
    torch.cuda.synchronize()
    rng = np.random.default_rng(2210 + N)
    for m, d in zip(mats, host):
        rows = np.unique(np.concatenate([rng.integers(0, m.M, 500), np.arange(m.M - 16, m.M), [0]]))
        yr, ar = oracle.gemm_nvfp4(d.codes, d.scales, d.g, d.x, rows=rows)
        assert_close(m.y.cpu().numpy()[:, rows], yr, ar, "valu M=%d K=%d N=%d" % (m.M, m.K, N))


def test_valu_column_invariance_and_ragged_shapes(wq):
    specs = [(96, 17408), (40, 17440), (33, 8736), (17, 544), (1, 32)]
    host = [inputs.nvfp4_inputs(M, K, 8, seed=2300 + i, g=0.02) for i, (M, K) in enumerate(specs)]
    tiled = [to_tiled(wq, d) for d in host]
    xs = [dev_bf16bits(d.x) for d in host]
    outs = {}
    for N in (1, 3, 8):
        mats = []
        for d, t, x in zip(host, tiled, xs):
            y = torch.full((N, d.M), float("nan"), dtype=torch.float32, device=DEV)
            mats.append(wq.Matrix(wq.WQ_FMT_NVFP4_TILED, d.M, d.K, t, None, x[:N].contiguous(), y, d.g))
        ws = workspace(wq.wq_verify_workspace_bytes(mats, N))
        plan = wq.wq_verify_prepare(mats, N, ws)
        print("valu column invariance N=%d" % N, flush=True)
        wq.wq_verify_launch_valu(plan)
        torch.cuda.synchronize()
        outs[N] = [m.y.cpu().numpy() for m in mats]
    for i, d in enumerate(host):
        yr, ar = oracle.gemm_nvfp4(d.codes, d.scales, d.g, d.x)
        assert_close(outs[8][i], yr, ar, "valu M=%d K=%d N=8" % (d.M, d.K))
        for N in (1, 3):
            assert np.array_equal(outs[N][i].view(np.uint32), outs[8][i][:N].view(np.uint32)), \
                "M=%d K=%d: N=%d differs from N=8" % (d.M, d.K, N)


def test_valu_rejects_non_tiled_plans(wq):
    d = inputs.nvfp4_inputs(64, 256, 2, seed=2400, g=0.02)
    y = torch.zeros((2, 64), dtype=torch.float32, device=DEV)
    m = wq.Matrix(wq.WQ_FMT_NVFP4, 64, 256, dev_u8(d.codes), dev_u8(d.scales), dev_bf16bits(d.x), y, d.g)
    ws = workspace(wq.wq_verify_workspace_bytes([m], 2))
    plan = wq.wq_verify_prepare([m], 2, ws)
    with pytest.raises(wq.WQError):
        wq.wq_verify_launch_valu(plan)
