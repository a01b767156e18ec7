"""The verify pass with a device-side column count, and in HIP graphs, on
the GPU through the C ABI: wq_verify_launch_n gives, for every n, the bits
a plan prepared for N = n gives and leaves rows n..7 alone; captured in a
graph (torch.cuda.CUDAGraph) it follows the count written between replays,
and a captured fixed-N pass replays to the same bits every time, with the
program's own eager work between the replays."""
import numpy as np
import pytest
import torch

import oracle
from fp8_weight_streaming_amd import inputs
from gpu_util import DEV, assert_close, dev_bf16bits, dev_f32, dev_u8, workspace

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def wq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from fp8_weight_streaming_amd import wq as mod
    return mod


@pytest.fixture(scope="module")
def tiled_pass(wq):
    # tiled NVFP4 (one matrix split in K, with a ragged last chunk) and tiled FP8
    mats, host, keep = [], [], []
    for i, (M, K) in enumerate([(300, 5120), (96, 17440), (160, 1056)]):
        d = inputs.nvfp4_inputs(M, K, 8, seed=1800 + i, g=0.02)
        t = torch.empty(wq.wq_nvfp4_tiled_bytes(M, K), dtype=torch.uint8, device=DEV)
        wq.wq_nvfp4_tile(dev_u8(d.codes), dev_u8(d.scales), t)
        x = dev_bf16bits(d.x)
        y = torch.full((8, M), float("nan"), dtype=torch.float32, device=DEV)
        mats.append((wq.WQ_FMT_NVFP4_TILED, M, K, t, None, x, y, d.g))
        host.append(("nvfp4", d))
    for i, (M, K) in enumerate([(2000, 1024), (50, 17424)]):
        d = inputs.fp8row_inputs(M, K, 8, seed=1810 + i)
        t = torch.empty(wq.wq_fp8_tiled_bytes(M, K), dtype=torch.uint8, device=DEV)
        wq.wq_fp8_tile(dev_u8(d.w), t)
        x, rs = dev_bf16bits(d.x), dev_f32(d.row_scale)
        y = torch.full((8, M), float("nan"), dtype=torch.float32, device=DEV)
        mats.append((wq.WQ_FMT_FP8ROW_TILED, M, K, t, rs, x, y, 1.0))
        host.append(("fp8", d))
    torch.cuda.synchronize()
    return mats, host


def plan_for(wq, mats, N):
    ms = [wq.Matrix(f, M, K, t, s, x[:N], y[:N], g) for (f, M, K, t, s, x, y, g) in mats]
    ws = workspace(wq.wq_verify_workspace_bytes(ms, N))
    return wq.wq_verify_prepare(ms, N, ws), ws


def outputs(mats):
    return [y.cpu().numpy().copy() for (*_, y, _g) in mats]


def reset(mats):
    for (*_, y, _g) in mats:
        y.fill_(float("nan"))


@pytest.fixture(scope="module")
def static_results(wq, tiled_pass):
    mats, host = tiled_pass
    res = {}
    for n in range(1, 9):
        reset(mats)
        plan, ws = plan_for(wq, mats, n)
        wq.wq_verify_launch(plan)
        torch.cuda.synchronize()
        res[n] = outputs(mats)
    # the static results themselves against the oracle, at N = 8
    for yo, (fmt, d) in zip(res[8], host):
        if fmt == "nvfp4":
            yr, ar = oracle.gemm_nvfp4(d.codes, d.scales, d.g, d.x)
        else:
            yr, ar = oracle.gemm_fp8row(d.w, d.row_scale, d.x)
        assert_close(yo, yr, ar, "static pass %s M=%d" % (fmt, d.M))
    return res


def check_n(res, n, got):
    for a, b in zip(got, res[n]):
        assert np.array_equal(a[:n].view(np.uint32), b[:n].view(np.uint32)), "n=%d bits" % n
        assert np.isnan(a[n:]).all(), "n=%d: rows past n were written" % n


def test_device_n_matches_static_plans(wq, tiled_pass, static_results):
    mats, _ = tiled_pass
    plan8, ws8 = plan_for(wq, mats, 8)
    n_dev = torch.zeros(1, dtype=torch.int32, device=DEV)
    for n in (3, 1, 8, 5, 2, 7, 4, 6):
        reset(mats)
        n_dev.fill_(n)
        print("device n=%d" % n, flush=True)
        wq.wq_verify_launch_n(plan8, n_dev)
        torch.cuda.synchronize()
        check_n(static_results, n, outputs(mats))


def test_graph_replays_follow_the_device_count(wq, tiled_pass, static_results):
    mats, _ = tiled_pass
    plan8, ws8 = plan_for(wq, mats, 8)
    n_dev = torch.full((1,), 8, dtype=torch.int32, device=DEV)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        wq.wq_verify_launch_n(plan8, n_dev, stream)   # eager first launch, outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        wq.wq_verify_launch_n(plan8, n_dev, stream)
    torch.cuda.synchronize()
    scratch = torch.ones(1 << 20, device=DEV)
    for n in (2, 8, 5, 3, 8, 1):
        reset(mats)
        n_dev.fill_(n)
        scratch.mul_(1.0001)          # the program's own work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        check_n(static_results, n, outputs(mats))


def test_graph_of_a_fixed_n_pass_replays_to_the_same_bits(wq, tiled_pass, static_results):
    mats, _ = tiled_pass
    plan4, ws4 = plan_for(wq, mats, 4)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        wq.wq_verify_launch(plan4, stream)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        wq.wq_verify_launch(plan4, stream)
    torch.cuda.synchronize()
    for _ in range(4):
        reset(mats)
        torch.randn(1 << 16, device=DEV).sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        check_n(static_results, 4, outputs(mats))
