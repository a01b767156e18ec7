"""Greedy draft acceptance fused onto the head product, on the GPU, through
the C ABI: the per-column tokens equal the oracle's greedy choice over the
kernel's own FP32 logits (an integer result, so exactly), the accepted
count equals the oracle's, the logits match the FP64 oracle within the
tolerance, and where the FP64 oracle's greedy row differs the two rows'
exact logits lie within the tolerance of each other."""
import numpy as np
import pytest
import torch

import oracle
from oracle.accept import greedy_accept, greedy_token
from fp8_weight_streaming_amd import inputs
from gpu_util import DEV, TOL, assert_close, dev_bf16bits, dev_f32, dev_u8, workspace

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def wq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from fp8_weight_streaming_amd import wq as mod
    return mod


def tiled_head(wq, d, fmt):
    if fmt == wq.WQ_FMT_FP8ROW_TILED:
        t = torch.empty(wq.wq_fp8_tiled_bytes(d.M, d.K), dtype=torch.uint8, device=DEV)
        wq.wq_fp8_tile(dev_u8(d.w), t)
        return t, dev_f32(d.row_scale), 1.0
    t = torch.empty(wq.wq_nvfp4_tiled_bytes(d.M, d.K), dtype=torch.uint8, device=DEV)
    wq.wq_nvfp4_tile(dev_u8(d.codes), dev_u8(d.scales), t)
    return t, None, d.g


def run_accept(wq, fmt, head, d, N, drafts, with_logits=True):
    t, rs, g = head
    x = dev_bf16bits(d.x[:N])
    dr = torch.tensor(list(drafts) if N > 1 else [0], dtype=torch.int32, device=DEV)
    logits = torch.full((N, d.M), float("nan"), dtype=torch.float32, device=DEV) if with_logits else None
    tokens = torch.full((N,), -7, dtype=torch.int32, device=DEV)
    acc = torch.full((1,), -7, dtype=torch.int32, device=DEV)
    ws = workspace(wq.wq_head_accept_workspace_bytes(fmt, d.M, d.K, N))
    wq.wq_head_accept(fmt, t, rs, g, x, d.M, d.K, dr, tokens, acc, logits=logits, workspace=ws)
    torch.cuda.synchronize()
    return (tokens.cpu().numpy(), int(acc.cpu().numpy()[0]),
            None if logits is None else logits.cpu().numpy())


def oracle_gemm(fmt_name, d, N, rows=None):
    if fmt_name == "fp8":
        return oracle.gemm_fp8row(d.w, d.row_scale, d.x[:N], rows=rows)
    return oracle.gemm_nvfp4(d.codes, d.scales, d.g, d.x[:N], rows=rows)


def check_round(wq, fmt, fmt_name, head, d, N, rng):
    # first run: any drafts, to learn the tokens; then drafts that are all
    # accepted, accepted up to a random point, and wrong from the start
    tok0, _, lg = run_accept(wq, fmt, head, d, N, [0] * (N - 1))
    yr, ar = oracle_gemm(fmt_name, d, N)
    assert_close(lg, yr, ar, "head logits %s M=%d K=%d N=%d" % (fmt_name, d.M, d.K, N))
    for n in range(N):
        assert tok0[n] == greedy_token(lg[n]), "column %d: kernel token vs greedy over its logits" % n
        r = greedy_token(yr[n])
        if r != tok0[n]:   # FP32 rounding may reorder near-equal logits: both must be near the top
            assert abs(yr[n][r] - yr[n][tok0[n]]) <= TOL * (ar[n][r] + ar[n][tok0[n]]), "column %d" % n
    patterns = [list(tok0[:N - 1])]
    if N > 1:
        j = int(rng.integers(0, N - 1))
        bad = list(tok0[:N - 1])
        bad[j] = (bad[j] + 1) % d.M
        patterns += [bad, [(int(tok0[0]) + 3) % d.M] + list(tok0[1:N - 1])]
    for drafts in patterns:
        tok, a, lg2 = run_accept(wq, fmt, head, d, N, drafts)
        assert np.array_equal(tok, tok0) and np.array_equal(lg2.view(np.uint32), lg.view(np.uint32))
        assert a == greedy_accept(lg2, drafts)[1], "drafts %s tokens %s accepted %d" % (drafts, tok, a)
    tok3, a3, _ = run_accept(wq, fmt, head, d, N, patterns[-1], with_logits=False)
    assert np.array_equal(tok3, tok0) and a3 == greedy_accept(lg, patterns[-1])[1]


@pytest.mark.parametrize("N", [1, 2, 3, 5, 8])
def test_fp8_head_accept(wq, N):
    d = inputs.fp8row_inputs(20011, 1024, 8, seed=1500 + N)
    head = tiled_head(wq, d, wq.WQ_FMT_FP8ROW_TILED)
    check_round(wq, wq.WQ_FMT_FP8ROW_TILED, "fp8", head, d, N, np.random.default_rng(N))


@pytest.mark.parametrize("N", [2, 8])
def test_nvfp4_head_accept(wq, N):
    d = inputs.nvfp4_inputs(9001, 5120, 8, seed=1600 + N, g=0.02)
    head = tiled_head(wq, d, wq.WQ_FMT_NVFP4_TILED)
    check_round(wq, wq.WQ_FMT_NVFP4_TILED, "nvfp4", head, d, N, np.random.default_rng(10 + N))


def test_head_accept_ties_and_nan(wq):
    N = 8
    d = inputs.fp8row_inputs(5000, 512, N, seed=1700)
    # a row far above the rest for every column: E4M3 448 with the sign of
    # column 0's X, copied to rows 37 and 37 + 16 * 200 (same place in their
    # tiles, so the same sums bit for bit): the lower row must win
    sign = (inputs.bf16_to_f32(d.x[0]) < 0).astype(np.uint8) << 7
    top = (0x7E | sign).astype(np.uint8)
    for m in (37 + 16 * 200, 37):
        d.w[m] = top
        d.row_scale[m] = 1.0
    head = tiled_head(wq, d, wq.WQ_FMT_FP8ROW_TILED)
    tok, a, lg = run_accept(wq, wq.WQ_FMT_FP8ROW_TILED, head, d, N, [37] * (N - 1))
    assert lg[0, 37] == lg[0, 37 + 16 * 200] and tok[0] == 37
    assert all(tok[n] == greedy_token(lg[n]) for n in range(N))
    assert a == greedy_accept(lg, [37] * (N - 1))[1]
    # NaN codes in rows 4000 and 123: every column's token is row 123
    d.w[4000, 9] = 0x7F
    d.w[123, 500] = 0xFF
    head = tiled_head(wq, d, wq.WQ_FMT_FP8ROW_TILED)
    tok, a, lg = run_accept(wq, wq.WQ_FMT_FP8ROW_TILED, head, d, N, [123, 123, 5, 0, 0, 0, 0])
    assert np.isnan(lg[:, 123]).all() and np.isnan(lg[:, 4000]).all()
    assert (tok == 123).all() and a == 2


def test_head_accept_full_fp8_head(wq):
    # the 151936 x 5120 FP8 head at N = 8
    wl = inputs.workload(4)
    s = wl.matrices[0]
    d = inputs.fp8row_inputs(s.M, s.K, 8, wl.seed(0))
    head = tiled_head(wq, d, wq.WQ_FMT_FP8ROW_TILED)
    tok, _, lg = run_accept(wq, wq.WQ_FMT_FP8ROW_TILED, head, d, 8, [0] * 7)
    drafts = list(tok[:7])
    drafts[5] = (drafts[5] + 1) % s.M
    tok2, a, lg2 = run_accept(wq, wq.WQ_FMT_FP8ROW_TILED, head, d, 8, drafts)
    assert np.array_equal(tok, tok2) and a == 5
    for n in range(8):
        assert tok[n] == greedy_token(lg[n])
    # the kernel's rows against the FP64 oracle on those rows and its own best rows
    rows = np.unique(tok)
    yr, ar = oracle.gemm_fp8row(d.w, d.row_scale, d.x, rows=rows)
    assert_close(lg[:, rows], yr, ar, "full head at the chosen rows")
