"""Tiled NVFP4 and tiled FP8-row on the GPU: the conversion kernels match
the layouts' numpy statements byte for byte and invert exactly; the tiled
products match the oracle, and the plain products bit for bit when both use
the same K split."""
import numpy as np
import pytest
import torch

import oracle
from fp8_weight_streaming_amd import inputs
from gpu_util import DEV, assert_close, dev_bf16bits, dev_f32, dev_u8, run_fp8, run_nvfp4, workspace
from tiled_ref import fp8_tile_ref, tile_ref

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


# ---- tiled FP8-row ------------------------------------------------------------

def to_fp8_tiled(wq, d):
    t = torch.empty(wq.wq_fp8_tiled_bytes(d.M, d.K), dtype=torch.uint8, device=DEV)
    wq.wq_fp8_tile(dev_u8(d.w), t)
    return t


def run_fp8_tiled(wq, d, N, x=None):
    x = d.x if x is None else x
    t = to_fp8_tiled(wq, d)
    y = torch.full((N, d.M), float("nan"), dtype=torch.float32, device=DEV)
    ws = workspace(wq.wq_gemm_workspace_bytes(wq.WQ_FMT_FP8ROW_TILED, d.M, d.K, N))
    wq.wq_gemm_fp8row_tiled(t, dev_f32(d.row_scale), dev_bf16bits(x[:N]), y, d.M, d.K, ws)
    torch.cuda.synchronize()
    return y.cpu().numpy()


FP8_SHAPES = [(1, 16), (16, 128), (17, 48), (33, 208), (100, 544), (64, 1024), (250, 4240), (48, 8720),
              (40, 17424), (5000, 5120)]


@pytest.mark.parametrize("M,K", FP8_SHAPES)
def test_fp8_tile_matches_layout_and_inverts(wq, M, K):
    d = inputs.fp8row_inputs(M, K, 1, seed=500 + M + K)
    t = to_fp8_tiled(wq, d)
    torch.cuda.synchronize()
    assert np.array_equal(t.cpu().numpy(), fp8_tile_ref(d.w)), "tiled bytes differ"
    w = torch.zeros((M, K), dtype=torch.uint8, device=DEV)
    wq.wq_fp8_untile(t, w)
    torch.cuda.synchronize()
    assert np.array_equal(w.cpu().numpy(), d.w)


@pytest.mark.parametrize("M,K", FP8_SHAPES[:-1])
def test_fp8_tiled_gemm_all_n(wq, M, K):
    d = inputs.fp8row_inputs(M, K, 8, seed=600 + M + K)
    same = wq.wq_gemm_split(wq.WQ_FMT_FP8ROW, M, K) == wq.wq_gemm_split(wq.WQ_FMT_FP8ROW_TILED, M, K)
    print("M=%d K=%d split plain=%s tiled=%s" % (M, K, wq.wq_gemm_split(1, M, K), wq.wq_gemm_split(3, M, K)),
          flush=True)
    for N in range(1, 9):
        y = run_fp8_tiled(wq, d, N)
        yr, ar = oracle.gemm_fp8row(d.w, d.row_scale, d.x[:N])
        assert_close(y, yr, ar, "fp8 tiled M=%d K=%d N=%d" % (M, K, N))
        if same:
            yp = run_fp8(wq, d, N)
            assert np.array_equal(yp.view(np.uint32), y.view(np.uint32)), "fp8 tiled vs plain bits N=%d" % N


def test_fp8_tiled_edge_values(wq):
    # NaN codes (S.1111.111) propagate only to their row; a zero row scale gives zeros
    d = inputs.fp8row_inputs(40, 256, 8, seed=77)
    d.w[3, 5] = 0x7F
    d.w[21, 200] = 0xFF
    d.row_scale[9] = 0.0
    y = run_fp8_tiled(wq, d, 8)
    yr, ar = oracle.gemm_fp8row(d.w, d.row_scale, d.x)
    assert_close(y, yr, ar, "fp8 tiled edge values")
    assert np.isnan(y[:, 3]).all() and np.isnan(y[:, 21]).all() and (y[:, 9] == 0).all()


def test_fp8_tiled_column_invariance(wq):
    d = inputs.fp8row_inputs(96, 17424, 8, seed=19)
    y8 = run_fp8_tiled(wq, d, 8)
    for N in (1, 3, 5, 7):
        assert np.array_equal(run_fp8_tiled(wq, d, N).view(np.uint32), y8[:N].view(np.uint32))


@pytest.mark.parametrize("N", [2, 8])
def test_tiled_pass_nvfp4_and_fp8(wq, N):
    # a dense layer in tiled NVFP4 next to a tiled FP8-row head slice, in one launch
    mats, host, keep = [], [], []
    for i, s in enumerate(inputs.VERIFY_LAYER):
        d = inputs.nvfp4_inputs(s.M, s.K, N, seed=1300 + i, g=0.02)
        t = to_tiled(wq, d)
        y = torch.full((N, s.M), float("nan"), dtype=torch.float32, device=DEV)
        x = dev_bf16bits(d.x)
        mats.append(wq.Matrix(wq.WQ_FMT_NVFP4_TILED, s.M, s.K, t, None, x, y, d.g))
        host.append(("nvfp4", d))
        keep.append((t, x))
    d = inputs.fp8row_inputs(20000, 5120, N, seed=1310)
    t, rs, x = to_fp8_tiled(wq, d), dev_f32(d.row_scale), dev_bf16bits(d.x)
    y = torch.full((N, d.M), float("nan"), dtype=torch.float32, device=DEV)
    mats.append(wq.Matrix(wq.WQ_FMT_FP8ROW_TILED, d.M, d.K, t, rs, x, y, 1.0))
    host.append(("fp8", d))
    keep.append((t, rs, x))
    ws = workspace(wq.wq_verify_workspace_bytes(mats, N))
    wq.wq_verify_pass(mats, N, ws)
    torch.cuda.synchronize()
    rng = np.random.default_rng(88 + N)
    for m, (fmt, d) in zip(mats, host):
        rows = np.unique(np.concatenate([rng.integers(0, m.M, 400), [0, m.M - 1]]))
        if fmt == "nvfp4":
            yr, ar = oracle.gemm_nvfp4(d.codes, d.scales, d.g, d.x, rows=rows)
        else:
            yr, ar = oracle.gemm_fp8row(d.w, d.row_scale, d.x, rows=rows)
        assert_close(m.y.cpu().numpy()[:, rows], yr, ar, "tiled pass %s M=%d K=%d N=%d" % (fmt, m.M, m.K, N))


def test_mixed_pass_plain_and_tiled(wq):
    # every format in one launch (the mixed kernel), small shapes with ragged tails
    N = 5
    mats, host, keep = [], [], []
    dn = inputs.nvfp4_inputs(100, 544, N, seed=1400, g=0.02)
    mats.append(wq.Matrix(wq.WQ_FMT_NVFP4, dn.M, dn.K, dev_u8(dn.codes), dev_u8(dn.scales), dev_bf16bits(dn.x),
                          torch.full((N, dn.M), float("nan"), dtype=torch.float32, device=DEV), dn.g))
    host.append(("nvfp4", dn))
    dt = inputs.nvfp4_inputs(33, 17440, N, seed=1401, g=0.02)
    mats.append(wq.Matrix(wq.WQ_FMT_NVFP4_TILED, dt.M, dt.K, to_tiled(wq, dt), None, dev_bf16bits(dt.x),
                          torch.full((N, dt.M), float("nan"), dtype=torch.float32, device=DEV), dt.g))
    host.append(("nvfp4", dt))
    df = inputs.fp8row_inputs(70, 208, N, seed=1402)
    mats.append(wq.Matrix(wq.WQ_FMT_FP8ROW, df.M, df.K, dev_u8(df.w), dev_f32(df.row_scale), dev_bf16bits(df.x),
                          torch.full((N, df.M), float("nan"), dtype=torch.float32, device=DEV), 1.0))
    host.append(("fp8", df))
    dg = inputs.fp8row_inputs(50, 17424, N, seed=1403)
    mats.append(wq.Matrix(wq.WQ_FMT_FP8ROW_TILED, dg.M, dg.K, to_fp8_tiled(wq, dg), dev_f32(dg.row_scale),
                          dev_bf16bits(dg.x), torch.full((N, dg.M), float("nan"), dtype=torch.float32, device=DEV),
                          1.0))
    host.append(("fp8", dg))
    ws = workspace(wq.wq_verify_workspace_bytes(mats, N))
    wq.wq_verify_pass(mats, N, ws)
    torch.cuda.synchronize()
    for m, (fmt, d) in zip(mats, host):
        if fmt == "nvfp4":
            yr, ar = oracle.gemm_nvfp4(d.codes, d.scales, d.g, d.x)
        else:
            yr, ar = oracle.gemm_fp8row(d.w, d.row_scale, d.x)
        assert_close(m.y.cpu().numpy(), yr, ar, "mixed pass fmt=%d M=%d K=%d" % (m.fmt, m.M, m.K))


@pytest.mark.parametrize("fmt", ["nvfp4", "fp8", "nvfp4-ksplit"])
def test_short_runs_write_held_outputs(wq, fmt):
    # Single tiled products with at least 8 row tiles per CU run the stream
    # kernel, here with one or two tiles per wave: from N = 4 up each wave's
    # output pairs wait in LDS until its run ends.  Ragged M (NVFP4: a last
    # tile of one row at an even index, written alone; FP8: 15 rows at an
    # odd index) and ragged K.  Every output (reset to NaN) must match the
    # oracle, and each column the N = 1 product (whose outputs are written as
    # they come) bit for bit.  nvfp4-ksplit: K = 10240 in two chunks of 5120,
    # so the held pairs are chunk sums written to the partial planes that a
    # reduction then adds.
    if fmt == "nvfp4-ksplit":
        d = inputs.nvfp4_inputs(36001, 10240, 8, seed=2102, g=0.02)
        run = run_tiled
        yr, ar = oracle.gemm_nvfp4(d.codes, d.scales, d.g, d.x)
    elif fmt == "nvfp4":
        d = inputs.nvfp4_inputs(36001, 544, 8, seed=2100, g=0.02)
        run = run_tiled
        yr, ar = oracle.gemm_nvfp4(d.codes, d.scales, d.g, d.x)
    else:
        d = inputs.fp8row_inputs(35999, 272, 8, seed=2101)
        run = run_fp8_tiled
        yr, ar = oracle.gemm_fp8row(d.w, d.row_scale, d.x)
    y1 = run(wq, d, 1)
    for N in (4, 5, 8):
        print("held outputs %s M=%d K=%d N=%d" % (fmt, d.M, d.K, N), flush=True)
        y = run(wq, d, N)
        assert_close(y, yr[:N], ar[:N], "held outputs %s N=%d" % (fmt, N))
        assert np.array_equal(y[:1].view(np.uint32), y1.view(np.uint32)), "column 0 differs from N = 1, N=%d" % N


@pytest.mark.parametrize("N", [3, 8])
def test_dynamic_tail_covers_every_unit_on_every_launch(wq, N):
    # A pass large enough (>= 256 units per workgroup) for the dynamic tail:
    # two tiled matrices, so the tail crosses a matrix boundary.  Every output
    # of every one of three launches (outputs reset to NaN in between) must
    # match the oracle: a chunk claimed twice or never would show, and so
    # would a claim counter that left a launch in the wrong state for the
    # next.  Then the plan is prepared again into the same workspace (the
    # counter starts over at zero) and two more launches must give the same
    # bits.  (At N = 8 the tail claims' outputs wait in LDS until each claim
    # ends.)
    specs = [(600000, 256), (500000, 256)]
    host = [inputs.nvfp4_inputs(M, K, N, seed=1900 + i, g=0.02) for i, (M, K) in enumerate(specs)]
    mats = []
    for d in host:
        t = to_tiled(wq, d)
        y = torch.full((N, d.M), float("nan"), dtype=torch.float32, device=DEV)
        mats.append(wq.Matrix(wq.WQ_FMT_NVFP4_TILED, d.M, d.K, t, None, dev_bf16bits(d.x), y, d.g))
    ws = workspace(wq.wq_verify_workspace_bytes(mats, N))
    plan = wq.wq_verify_prepare(mats, N, ws)
    refs = [oracle.gemm_nvfp4(d.codes, d.scales, d.g, d.x) for d in host]
    for launch in range(3):
        for m in mats:
            m.y.fill_(float("nan"))
        print("tail launch %d N=%d" % (launch, N), flush=True)
        wq.wq_verify_launch(plan)
        torch.cuda.synchronize()
        for m, (yr, ar) in zip(mats, refs):
            assert_close(m.y.cpu().numpy(), yr, ar, "launch %d M=%d" % (launch, m.M))
    last = [m.y.clone() for m in mats]
    plan = wq.wq_verify_prepare(mats, N, ws)
    for launch in range(2):
        for m in mats:
            m.y.fill_(float("nan"))
        print("tail launch %d after a new prepare N=%d" % (launch, N), flush=True)
        wq.wq_verify_launch(plan)
        torch.cuda.synchronize()
        for m, y0 in zip(mats, last):
            assert torch.equal(m.y.view(torch.int32), y0.view(torch.int32)), "after a new prepare M=%d" % m.M


def test_blocked_split_pass(wq):
    # A pass large enough that its split matrices (tiled NVFP4, K = 8736, and
    # tiled FP8-row, K = 8720: two K chunks each, ragged last tiles) are
    # computed in blocks of tiles whose chunk sums stay in LDS, with no
    # partial sums in the workspace and no reduction launch, ahead of a third
    # matrix that holds the dynamic tail (the planner's host test covers tail
    # claims inside blocked matrices).  Every launch of three
    # (outputs reset to NaN in between) must match the oracle on sampled rows,
    # equal the single-matrix products (which add the same chunk sums in a
    # reduction kernel) bit for bit when the splits agree, and column n must
    # not depend on N (N = 1, 3, 5 against 8: different block sizes).
    host = [("nvfp4", inputs.nvfp4_inputs(150007, 8736, 8, seed=1950, g=0.02)),
            ("fp8", inputs.fp8row_inputs(60011, 8720, 8, seed=1951)),
            ("nvfp4", inputs.nvfp4_inputs(700000, 256, 8, seed=1952, g=0.02))]
    tiled = [to_tiled(wq, d) if f == "nvfp4" else to_fp8_tiled(wq, d) for f, d in host]
    xs = [dev_bf16bits(d.x) for _, d in host]
    rss = [dev_f32(d.row_scale) if f == "fp8" else None for f, d in host]
    outs = {}
    for N in (1, 3, 5, 8):
        mats = []
        for (f, d), t, x, rs in zip(host, tiled, xs, rss):
            y = torch.full((N, d.M), float("nan"), dtype=torch.float32, device=DEV)
            if f == "nvfp4":
                mats.append(wq.Matrix(wq.WQ_FMT_NVFP4_TILED, d.M, d.K, t, None, x[:N].contiguous(), y, d.g))
            else:
                mats.append(wq.Matrix(wq.WQ_FMT_FP8ROW_TILED, d.M, d.K, t, rs, x[:N].contiguous(), y, 1.0))
        ws = workspace(wq.wq_verify_workspace_bytes(mats, N))
        plan = wq.wq_verify_prepare(mats, N, ws)
        print("blocked pass N=%d: reduce runs %d, lds_extra %d" % (N, plan.reduce_runs, plan.lds_extra), flush=True)
        assert plan.reduce_runs == 0 and plan.lds_extra > 0
        rng = np.random.default_rng(1960 + N)
        refs = []
        for f, d in host:
            rows = np.unique(np.concatenate([rng.integers(0, d.M, 600), np.arange(d.M - 16, d.M), [0]]))
            if f == "nvfp4":
                refs.append((rows,) + oracle.gemm_nvfp4(d.codes, d.scales, d.g, d.x[:N], rows=rows))
            else:
                refs.append((rows,) + oracle.gemm_fp8row(d.w, d.row_scale, d.x[:N], rows=rows))
        for launch in range(3):
            for m in mats:
                m.y.fill_(float("nan"))
            print("blocked pass N=%d launch %d" % (N, launch), flush=True)
            wq.wq_verify_launch(plan)
            torch.cuda.synchronize()
            for m, (rows, yr, ar) in zip(mats, refs):
                assert_close(m.y.cpu().numpy()[:, rows], yr, ar, "N=%d launch %d M=%d K=%d" % (N, launch, m.M, m.K))
        outs[N] = [m.y.cpu().numpy() for m in mats]
        if N == 8:
            # the same plan with the NVFP4 steps on the vector ALUs (blocked
            # epilogue included)
            for m in mats:
                m.y.fill_(float("nan"))
            print("blocked pass N=8, vector-ALU steps", flush=True)
            wq.wq_verify_launch_valu(plan)
            torch.cuda.synchronize()
            for m, (rows, yr, ar) in zip(mats, refs):
                assert_close(m.y.cpu().numpy()[:, rows], yr, ar, "valu N=8 M=%d K=%d" % (m.M, m.K))
    for i, (_, d) in enumerate(host):
        for N in (1, 3, 5):
            assert np.array_equal(outs[N][i].view(np.uint32), outs[8][i][:N].view(np.uint32)), "M=%d: N=%d differs" % (d.M, N)
    for i, (f, d) in enumerate(host[:2]):
        fmt = wq.WQ_FMT_NVFP4_TILED if f == "nvfp4" else wq.WQ_FMT_FP8ROW_TILED
        if wq.wq_gemm_split(fmt, d.M, d.K) == wq.wq_gemm_split(fmt, d.M, d.K, 2):
            y1 = run_tiled(wq, d, 8) if f == "nvfp4" else run_fp8_tiled(wq, d, 8)
            assert np.array_equal(y1.view(np.uint32), outs[8][i].view(np.uint32)), "%s M=%d" % (f, d.M)
        else:
            print("%s: single-matrix split differs: bitwise comparison skipped" % f, flush=True)


def test_blocked_split_three_chunks_dense_down_shape(wq):
    # The dense pass's own down-projection split: K = 17408 (tiled NVFP4) and
    # K = 17424 (tiled FP8-row) computed in blocks of three K chunks of 5888
    # (the last FP8 chunk ragged, 5648).  The middle chunk is the only one
    # that both adds to a tile's running sums kept in LDS and leaves them
    # there for the next chunk.  A third matrix holds the dynamic tail.  Four
    # N (1, 2, 4, 8), three launches each with the outputs reset to NaN in
    # between: sampled rows (the last 16 of each matrix included) against the
    # oracle, column n the same bits for every N, and the single-matrix
    # products bit for bit wherever they use the same split.
    host = [("nvfp4", inputs.nvfp4_inputs(200003, 17408, 8, seed=1970, g=0.02)),
            ("fp8", inputs.fp8row_inputs(40009, 17424, 8, seed=1971)),
            ("nvfp4", inputs.nvfp4_inputs(700000, 256, 8, seed=1972, g=0.02))]
    for f, d in host[:2]:
        fmt = wq.WQ_FMT_NVFP4_TILED if f == "nvfp4" else wq.WQ_FMT_FP8ROW_TILED
        assert wq.wq_gemm_split(fmt, d.M, d.K, 2) == (5888, 3), (f, wq.wq_gemm_split(fmt, d.M, d.K, 2))
    tiled = [to_tiled(wq, d) if f == "nvfp4" else to_fp8_tiled(wq, d) for f, d in host]
    xs = [dev_bf16bits(d.x) for _, d in host]
    rss = [dev_f32(d.row_scale) if f == "fp8" else None for f, d in host]
    outs = {}
    for N in (1, 2, 4, 8):
        mats = []
        for (f, d), t, x, rs in zip(host, tiled, xs, rss):
            y = torch.full((N, d.M), float("nan"), dtype=torch.float32, device=DEV)
            if f == "nvfp4":
                mats.append(wq.Matrix(wq.WQ_FMT_NVFP4_TILED, d.M, d.K, t, None, x[:N].contiguous(), y, d.g))
            else:
                mats.append(wq.Matrix(wq.WQ_FMT_FP8ROW_TILED, d.M, d.K, t, rs, x[:N].contiguous(), y, 1.0))
        ws = workspace(wq.wq_verify_workspace_bytes(mats, N))
        plan = wq.wq_verify_prepare(mats, N, ws)
        print("3-chunk blocked pass N=%d: reduce runs %d, lds_extra %d" % (N, plan.reduce_runs, plan.lds_extra),
              flush=True)
        assert plan.reduce_runs == 0 and plan.lds_extra > 0
        rng = np.random.default_rng(1980 + N)
        refs = []
        for f, d in host:
            rows = np.unique(np.concatenate([rng.integers(0, d.M, 600), np.arange(d.M - 16, d.M), [0]]))
            if f == "nvfp4":
                refs.append((rows,) + oracle.gemm_nvfp4(d.codes, d.scales, d.g, d.x[:N], rows=rows))
            else:
                refs.append((rows,) + oracle.gemm_fp8row(d.w, d.row_scale, d.x[:N], rows=rows))
        for launch in range(3):
            for m in mats:
                m.y.fill_(float("nan"))
            print("3-chunk blocked pass N=%d launch %d" % (N, launch), flush=True)
            wq.wq_verify_launch(plan)
            torch.cuda.synchronize()
            for m, (rows, yr, ar) in zip(mats, refs):
                assert_close(m.y.cpu().numpy()[:, rows], yr, ar, "N=%d launch %d M=%d K=%d" % (N, launch, m.M, m.K))
        outs[N] = [m.y.cpu().numpy() for m in mats]
        del mats, ws, plan
    for i, (_, d) in enumerate(host):
        for N in (1, 2, 4):
            assert np.array_equal(outs[N][i].view(np.uint32), outs[8][i][:N].view(np.uint32)), \
                "M=%d K=%d: N=%d differs from N=8" % (d.M, d.K, N)
    for i, (f, d) in enumerate(host[:2]):
        fmt = wq.WQ_FMT_NVFP4_TILED if f == "nvfp4" else wq.WQ_FMT_FP8ROW_TILED
        if wq.wq_gemm_split(fmt, d.M, d.K) == wq.wq_gemm_split(fmt, d.M, d.K, 2):
            y1 = run_tiled(wq, d, 8) if f == "nvfp4" else run_fp8_tiled(wq, d, 8)
            assert np.array_equal(y1.view(np.uint32), outs[8][i].view(np.uint32)), "%s M=%d" % (f, d.M)
        else:
            print("%s: single-matrix split %s differs from the blocked split: bitwise comparison skipped"
                  % (f, wq.wq_gemm_split(fmt, d.M, d.K)), flush=True)


def test_split_tile_calls_share_one_workspace(wq):
    """Single products of the split-tile kernel (few row tiles, K cut into
    several chunks whose parts the last workgroup to arrive adds) called
    back to back on ONE workspace, zeroed once: every call must read the
    parts of its own call (the shapes are small, so earlier calls' parts
    and counters are still in the caches), match the oracle, and leave the
    arrival counters at zero."""
    shapes = [(32, 16384), (48, 8736), (16, 4096), (40, 17440)]
    data = [inputs.nvfp4_inputs(M, K, 8, seed=700 + M + K, g=0.02) for M, K in shapes]
    plans = [wq.wq_gemm_split(wq.WQ_FMT_NVFP4_TILED, M, K) for M, K in shapes]
    print("split-tile shapes %s plans %s" % (shapes, plans), flush=True)
    assert all(kc == 0 for kc, _ in plans) and any(nc > 1 for _, nc in plans)
    tiled = [to_tiled(wq, d) for d in data]
    nbytes = max(wq.wq_gemm_workspace_bytes(wq.WQ_FMT_NVFP4_TILED, M, K, 8) for M, K in shapes)
    ws = workspace(nbytes)
    rng = np.random.default_rng(71)
    for rep in range(3):
        for (M, K), d, t in zip(shapes, data, tiled):
            N = (8, 3, 5)[rep]
            x = inputs.to_bf16(rng.standard_normal((N, K)).astype(np.float32))
            y = torch.full((N, M), float("nan"), dtype=torch.float32, device=DEV)
            wq.wq_gemm_nvfp4_tiled(t, d.g, dev_bf16bits(x), y, M, K, ws)
            torch.cuda.synchronize()
            yr, ar = oracle.gemm_nvfp4(d.codes, d.scales, d.g, x)
            assert_close(y.cpu().numpy(), yr, ar, "repeat %d M=%d K=%d N=%d" % (rep, M, K, N))
    counters = ws[:16384].cpu().numpy()
    assert not counters.any(), "arrival counters not left at zero"
