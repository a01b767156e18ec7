"""Chained MLP layers on the GPU (wq_mlp_chain_*), layer by layer against
the oracle (oracle/chain.py), each stage from the GPU's own input to it:

  a   = BF16(RMSNorm(h) * gamma)  against the oracle's normalization of h;
  s   = BF16(silu(g) * u)         against the oracle's products of the GPU's a;
  h'  = h + s . Wd^T              against the oracle's product of the GPU's s.

Bounds (derived from the arithmetic, written in each check):
  * a: both sides round once to BF16 from values that differ by FP32
    rounding (a few 2^-24 relative), so they agree except where that
    difference straddles a rounding boundary -- then by one BF16 step
    (<= 2^-7 |a|), in a small fraction of elements.
  * s: g and u carry the products' error, at most TOL * sum |w a| (the
    GEMM parity bound); silu' is at most 1.1 in magnitude; then each side
    rounds to BF16 once (together <= 2^-7 max(|s|)).
  * h': TOL * sum |w s| for the product, plus FP32 rounding of the sum.
Multi-layer calls must equal one-layer calls bit for bit, a column's
results must not depend on N, and a captured graph must replay the eager
bits."""
import numpy as np
import pytest
import torch

import oracle
from fp8_weight_streaming_amd import inputs
from gpu_util import DEV, TOL, dev_bf16bits, dev_f32, dev_u8
from oracle import chain

pytestmark = pytest.mark.gpu
EPS = 1e-6


@pytest.fixture(scope="module")
def wq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from fp8_weight_streaming_amd import wq as mod
    return mod


class Layer:
    """One layer's host inputs and device buffers."""

    def __init__(self, wq, D, F, seed):
        self.D, self.F = D, F
        self.inp = inputs.mlp_layer_inputs(D, F, seed, up_gain=1.37)
        g, u, d = self.inp.gate, self.inp.up, self.inp.down
        self.gate_up = torch.empty(wq.wq_nvfp4_tiled_bytes(2 * F, D), dtype=torch.uint8, device=DEV)
        wq.wq_nvfp4_tile_glu(dev_u8(g.codes), dev_u8(g.scales), dev_u8(u.codes), dev_u8(u.scales), self.gate_up)
        self.down = torch.empty(wq.wq_nvfp4_tiled_bytes(D, F), dtype=torch.uint8, device=DEV)
        wq.wq_nvfp4_tile(dev_u8(d.codes), dev_u8(d.scales), self.down)
        self.gamma = dev_bf16bits(self.inp.gamma)
        self.desc = wq.MlpLayer(self.gate_up, self.down, self.gamma, g.g, u.g, d.g)

    def tuples(self):
        t = lambda m: (m.codes, m.scales, m.g)
        return t(self.inp.gate), t(self.inp.up), t(self.inp.down)


def run_chain(wq, layers, h0, stream=None, persistent=False):
    """Runs the layers on columns h0 [N][D]; returns (h, a, s) as numpy
    (one launch per kernel, or the single cooperative launch)."""
    N, D = h0.shape
    F = layers[0].F
    h = dev_f32(h0)
    a = torch.full((N, D), -1, dtype=torch.int16, device=DEV)
    s = torch.full((N, F), -1, dtype=torch.int16, device=DEV)
    ws = torch.empty(wq.wq_mlp_chain_workspace_bytes(len(layers), D, F, N), dtype=torch.uint8, device=DEV)
    plan = wq.wq_mlp_chain_prepare([y.desc for y in layers], D, F, N, EPS, h, a, s, ws)
    if persistent:
        assert plan.grid_chain > 0
        wq.wq_mlp_chain_launch_persistent(plan)
    else:
        wq.wq_mlp_chain_launch(plan)
    torch.cuda.synchronize()
    if persistent:
        ctl = ws[plan.ctl_offset:plan.ctl_offset + 16].cpu().numpy().view(np.uint32)
        assert ctl[0] == 0 and ctl[2] == 0, "grid barrier state %s" % ctl.tolist()
    return (h.cpu().numpy(), a.cpu().numpy().view(np.uint16), s.cpu().numpy().view(np.uint16))


def check_layer(layer, h0, h1, a_bits, s_bits, what):
    """Checks one layer's GPU outputs (a, s, new h) against the oracle."""
    h0 = np.asarray(h0, np.float64)
    gate, up, down = layer.tuples()
    # a
    a_gpu = chain.bf16_value(a_bits)
    a_ref = chain.normalize(h0, layer.inp.gamma, EPS)
    diff = a_gpu != a_ref
    assert np.all(np.abs(a_gpu - a_ref) <= 2.0 ** -7 * np.abs(a_ref)), "%s: a off by more than a BF16 step" % what
    assert diff.mean() < 0.01, "%s: a differs in %.3f of elements" % (what, diff.mean())
    # s from the GPU's a
    g, ag = oracle.gemm_nvfp4(gate[0], gate[1], gate[2], a_bits)
    u, au = oracle.gemm_nvfp4(up[0], up[1], up[2], a_bits)
    s_ref = chain.bf16_round(chain.silu(g) * u)
    s_gpu = chain.bf16_value(s_bits)
    eg, eu = TOL * ag, TOL * au
    bound = 1.1 * np.abs(u) * eg + (np.abs(chain.silu(g)) + 1.1 * eg) * eu + 2.0 ** -7 * np.maximum(
        np.abs(s_ref), np.abs(s_gpu)) + 1e-37
    err = np.abs(s_gpu - s_ref)
    assert np.all(err <= bound), "%s: s outside its bound at %s" % (what, np.argwhere(err > bound)[:4].tolist())
    assert np.mean(s_gpu == s_ref) > 0.98, "%s: s equal in only %.3f" % (what, np.mean(s_gpu == s_ref))
    # h' from the GPU's s
    y, ay = oracle.gemm_nvfp4(down[0], down[1], down[2], s_bits)
    href = h0 + y
    bound = TOL * ay + 2.0 ** -23 * (np.abs(h0) + np.abs(y)) + 1e-37
    err = np.abs(np.asarray(h1, np.float64) - href)
    assert np.all(err <= bound), "%s: h outside its bound (worst %.3g of it)" % (what, (err / bound).max())


SMALL = [(32, 32), (64, 96), (320, 544), (1024, 4352)]


@pytest.mark.parametrize("D,F", SMALL)
@pytest.mark.parametrize("N", [1, 3, 8])
def test_one_layer_matches_oracle(wq, D, F, N):
    print("chain layer D=%d F=%d N=%d" % (D, F, N), flush=True)
    layer = Layer(wq, D, F, seed=D + F)
    h0 = inputs.residual_inputs(N, D, seed=7 + N)
    h1, a, s = run_chain(wq, [layer], h0)
    check_layer(layer, h0, h1, a, s, "D=%d F=%d N=%d" % (D, F, N))


def test_gate_up_tiling_is_the_interleave(wq):
    F, D = 40, 288
    g = inputs.nvfp4_inputs(F, D, 1, seed=5)
    u = inputs.nvfp4_inputs(F, D, 1, seed=6)
    t = torch.empty(wq.wq_nvfp4_tiled_bytes(2 * F, D), dtype=torch.uint8, device=DEV)
    wq.wq_nvfp4_tile_glu(dev_u8(g.codes), dev_u8(g.scales), dev_u8(u.codes), dev_u8(u.scales), t)
    # tile t: gate rows 8t..8t+7, then up rows 8t..8t+7
    order = np.concatenate([np.r_[8 * i:8 * i + 8] + off for i in range(F // 8) for off in (0, F)])
    codes = np.concatenate([g.codes, u.codes])[order]
    scales = np.concatenate([g.scales, u.scales])[order]
    ref = torch.empty_like(t)
    wq.wq_nvfp4_tile(dev_u8(codes), dev_u8(scales), ref)
    torch.cuda.synchronize()
    assert torch.equal(t, ref)


def test_layers_in_one_call_equal_one_call_per_layer(wq):
    D, F, N = 320, 544, 5
    layers = [Layer(wq, D, F, seed=40 + i) for i in range(3)]
    h0 = inputs.residual_inputs(N, D, seed=41)
    h = h0
    for i, y in enumerate(layers):
        h1, a, s = run_chain(wq, [y], h)
        check_layer(y, h, h1, a, s, "layer %d" % i)
        h = h1
    hc, ac, sc = run_chain(wq, layers, h0)
    assert np.array_equal(hc.view(np.uint32), h.view(np.uint32))
    assert np.array_equal(ac, a) and np.array_equal(sc, s)


def test_columns_do_not_depend_on_n(wq):
    D, F = 1024, 4352
    layers = [Layer(wq, D, F, seed=60 + i) for i in range(2)]
    h0 = inputs.residual_inputs(8, D, seed=61)
    h8, a8, s8 = run_chain(wq, layers, h0)
    for n in (1, 3, 6):
        hn, an, sn = run_chain(wq, layers, h0[:n])
        assert np.array_equal(hn.view(np.uint32), h8[:n].view(np.uint32)), n
        assert np.array_equal(an, a8[:n]) and np.array_equal(sn, s8[:n]), n


def test_repeat_is_bitwise_and_graph_replays(wq):
    D, F, N = 1024, 4352, 4
    layers = [Layer(wq, D, F, seed=80 + i) for i in range(2)]
    h0 = inputs.residual_inputs(N, D, seed=81)
    ref = run_chain(wq, layers, h0)
    assert all(np.array_equal(x.view(np.uint8), y.view(np.uint8)) for x, y in zip(ref, run_chain(wq, layers, h0)))
    # capture the launches (no host work, no allocation) and replay
    h = dev_f32(h0)
    a = torch.zeros((N, D), dtype=torch.int16, device=DEV)
    s = torch.zeros((N, F), dtype=torch.int16, device=DEV)
    ws = torch.empty(wq.wq_mlp_chain_workspace_bytes(2, D, F, N), dtype=torch.uint8, device=DEV)
    h_init = dev_f32(h0)
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        plan = wq.wq_mlp_chain_prepare([y.desc for y in layers], D, F, N, EPS, h, a, s, ws, stream=side)
    side.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        wq.wq_mlp_chain_launch(plan, stream=side)
    for rep in range(3):
        h.copy_(h_init)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(h.cpu().numpy().view(np.uint32), ref[0].view(np.uint32)), rep
        assert np.array_equal(s.cpu().numpy().view(np.uint16), ref[2]), rep


def test_full_size_layers(wq):
    # the dense MLP of the verify workload: D = 5120, F = 17408, N = 8
    D, F, N = 5120, 17408, 8
    print("chain full size D=%d F=%d N=%d" % (D, F, N), flush=True)
    layers = [Layer(wq, D, F, seed=100 + i) for i in range(2)]
    h0 = inputs.residual_inputs(N, D, seed=101)
    h1, a1, s1 = run_chain(wq, layers[:1], h0)
    check_layer(layers[0], h0, h1, a1, s1, "full layer 0")
    h2, a2, s2 = run_chain(wq, layers, h0)
    h2b, a2b, s2b = run_chain(wq, layers[1:], h1)
    assert np.array_equal(h2.view(np.uint32), h2b.view(np.uint32))
    check_layer(layers[1], h1, h2, a2, s2, "full layer 1")


def test_zero_down_weights_pass_the_residual_through(wq):
    D, F, N = 256, 256, 3
    layer = Layer(wq, D, F, seed=9)
    layer.down.zero_()      # zero codes and zero scales
    h0 = inputs.residual_inputs(N, D, seed=10)
    h1, a, s = run_chain(wq, [layer], h0)
    assert np.array_equal(h1.view(np.uint32), h0.view(np.uint32))
    a_ref = chain.normalize(h0, layer.inp.gamma, EPS)
    assert np.all(np.abs(chain.bf16_value(a) - a_ref) <= 2.0 ** -7 * np.abs(a_ref))
    assert np.any(s != 0)


# ---- the single-launch chain ------------------------------------------------------

@pytest.mark.parametrize("D,F,N,L", [(32, 32, 1, 1), (64, 96, 3, 2), (320, 544, 8, 3), (1024, 4352, 5, 2)])
def test_single_launch_equals_launch_per_kernel(wq, D, F, N, L):
    # small shapes leave most workgroups without units in a phase: they
    # must still take part in every grid barrier
    print("single-launch chain D=%d F=%d N=%d L=%d" % (D, F, N, L), flush=True)
    layers = [Layer(wq, D, F, seed=200 + 7 * i + D) for i in range(L)]
    h0 = inputs.residual_inputs(N, D, seed=201)
    ref = run_chain(wq, layers, h0)
    got = run_chain(wq, layers, h0, persistent=True)
    for x, y in zip(ref, got):
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8))


def test_single_launch_full_size_and_repeat(wq):
    D, F, N = 5120, 17408, 8
    print("single-launch chain full size", flush=True)
    layers = [Layer(wq, D, F, seed=300 + i) for i in range(3)]
    h0 = inputs.residual_inputs(N, D, seed=301)
    h1, a1, s1 = run_chain(wq, layers[:1], h0, persistent=True)
    check_layer(layers[0], h0, h1, a1, s1, "single-launch full layer 0")
    ref = run_chain(wq, layers, h0)
    for rep in range(2):
        got = run_chain(wq, layers, h0, persistent=True)
        for x, y in zip(ref, got):
            assert np.array_equal(x.view(np.uint8), y.view(np.uint8)), rep

