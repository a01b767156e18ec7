"""Pins of the chained-MLP oracle (oracle/chain.py) against facts fixed
outside it: torch's float32 -> bfloat16 cast and its float64 rms_norm,
silu and linear (independent library routines), weights decoded from the
E2M1 fixture and torch's E4M3 cast, closed-form rounding cases, and the
invariants of the layer.  Each stage is compared with the oracle's own
input to that stage, so that a slip in any one of them (a dropped
normalization, gate and up swapped, a transposed weight, a missing
residual, rounding done twice) fails here by itself.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as TF

from fp8_weight_streaming_amd import inputs
from golden_util import e2m1_table
from oracle import chain

E2M1 = np.array([float(e2m1_table()[c]) for c in range(16)], np.float64)
E4M3 = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def dense(m) -> np.ndarray:
    """Decoded NVFP4 weights [R][C] in float64 (fixture table x torch E4M3 x g)."""
    lo = m.codes & 0xF
    hi = m.codes >> 4
    codes = np.stack([lo, hi], axis=2).reshape(m.codes.shape[0], -1)
    scale = np.repeat(E4M3[m.scales], 16, axis=1)
    return E2M1[codes] * scale * float(np.float32(m.g))


def torch_bf16(v32: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(v32, np.float32)).to(torch.bfloat16)
    return t.to(torch.float64).numpy()


def as_tuple(m):
    return (m.codes, m.scales, m.g)


# ---- BF16 rounding -----------------------------------------------------------

def test_bf16_round_matches_torch_cast_on_float32():
    rng = np.random.default_rng(3)
    with np.errstate(over="ignore"):
        v = (rng.standard_normal(200000) * np.exp2(rng.integers(-140, 128, 200000))).astype(np.float32)
    # exact ties between neighbouring BF16 values, and their neighbours
    b = rng.integers(0, 0x7F7F, 20000).astype(np.uint32) << 16
    ties = (b | 0x8000).view(np.float32)
    v = np.concatenate([v, ties, -ties, np.nextafter(ties, np.float32(0)), np.nextafter(ties, np.float32(np.inf)),
                        np.array([0.0, -0.0, np.inf, -np.inf, 3.3895314e38, 3.4028235e38, 1e-45, -1e-45,
                                  1.1754942e-38], np.float32)])
    with np.errstate(over="ignore"):
        ref = torch_bf16(v)
    got = chain.bf16_round(v.astype(np.float64))
    assert np.array_equal(got, ref)
    assert np.array_equal(np.signbit(got), np.signbit(ref))
    assert np.isnan(chain.bf16_round(np.array([np.nan])))[0]


def test_bf16_round_is_a_single_rounding():
    # 1 + 2^-8 lies halfway between 1 and 1 + 2^-7: ties go to the even 1.0;
    # a hair above the tie must round up, which rounding first to FP32 (that
    # hair is below FP32's resolution) would lose
    one = 1.0
    assert chain.bf16_round(np.array([one + 2.0 ** -8]))[0] == 1.0
    assert chain.bf16_round(np.array([one + 2.0 ** -8 + 2.0 ** -40]))[0] == 1.0 + 2.0 ** -7
    assert chain.bf16_round(np.array([-(one + 2.0 ** -8 + 2.0 ** -40)]))[0] == -(1.0 + 2.0 ** -7)
    assert chain.bf16_round(np.array([one + 2.0 ** -8 - 2.0 ** -40]))[0] == 1.0
    # tie with an odd lower neighbour rounds up to the even one
    assert chain.bf16_round(np.array([one + 3 * 2.0 ** -8]))[0] == 1.0 + 2.0 ** -6
    # every midpoint of a run of BF16 neighbours, nudged both ways in FP64
    lo = (np.arange(0x3F80, 0x4100, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)
    hi = (np.arange(0x3F81, 0x4101, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)
    mid = (lo + hi) / 2
    assert np.array_equal(chain.bf16_round(mid + 2.0 ** -45), hi)
    assert np.array_equal(chain.bf16_round(mid - 2.0 ** -45), lo)


def test_bf16_bits_roundtrip():
    bits = np.arange(0, 0x7F80, 7, dtype=np.uint16)
    assert np.array_equal(chain.bf16_bits(chain.bf16_value(bits)), bits)


# ---- the elementwise stages -------------------------------------------------

def test_silu_against_torch():
    v = np.concatenate([np.linspace(-60, 60, 2001), [0.0, -0.0, 1e-30, -745.0, 800.0]])
    ref = TF.silu(torch.from_numpy(v)).numpy()
    got = chain.silu(v)
    assert np.allclose(got, ref, rtol=1e-14, atol=1e-300)
    # silu(v) - silu(-v) = v
    w = np.linspace(-30, 30, 301)
    assert np.allclose(chain.silu(w) - chain.silu(-w), w, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("eps", [0.0, 1e-6, 0.5])
def test_rmsnorm_against_torch(eps):
    rng = np.random.default_rng(7)
    h = rng.standard_normal((3, 96)) * np.array([[1.0], [1e-3], [40.0]])
    gamma = inputs.to_bf16((1 + 0.3 * rng.standard_normal(96)).astype(np.float32))
    w = torch.from_numpy(chain.bf16_value(gamma))
    ref = TF.rms_norm(torch.from_numpy(h), (96,), weight=w, eps=float(np.float32(eps))).numpy()
    assert np.allclose(chain.rmsnorm(h, gamma, eps), ref, rtol=1e-13, atol=0)


def test_normalize_rounds_once_from_fp64():
    # half a million elements: rounding through FP32 first changes about one
    # element in 2^16 (those within FP32 resolution of a BF16 tie)
    rng = np.random.default_rng(9)
    N, D = 8, 65536
    h = rng.standard_normal((N, D)) * 3.0
    gamma = inputs.to_bf16((1 + 0.3 * rng.standard_normal(D)).astype(np.float32))
    T = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float64))
    pre = TF.rms_norm(T(h), (D,), weight=T(chain.bf16_value(gamma)), eps=1e-6).numpy()
    ref = torch_bf16(pre.astype(np.float32))           # double rounding, for contrast
    got = chain.normalize(h, gamma, 1e-6)
    assert np.array_equal(got, chain.bf16_round(pre))
    assert 0 < np.count_nonzero(got != ref) < 100


# ---- the layer, stage by stage ------------------------------------------------

def test_mlp_layer_stages_against_torch():
    D, F, N = 64, 96, 3
    L = inputs.mlp_layer_inputs(D, F, 11)
    h = inputs.residual_inputs(N, D, 12).astype(np.float64)
    eps = 1e-6
    r = chain.mlp_layer(h, as_tuple(L.gate), as_tuple(L.up), as_tuple(L.down), L.gamma, eps)
    T = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float64))

    # a: torch's rms_norm, rounded once to BF16
    pre = TF.rms_norm(T(h), (D,), weight=T(chain.bf16_value(L.gamma)), eps=float(np.float32(eps))).numpy()
    a_ref = chain.bf16_round(pre)
    # (FP64 results of two routines differ in the last bits; one of them
    # lands on the other side of a BF16 rounding boundary with odds of about
    # 1e-13 per element, so the rounded values must agree exactly)
    assert np.array_equal(r["a"], a_ref)

    # g, u from the oracle's a; gate applies to the silu, up multiplies
    Wg, Wu, Wd = dense(L.gate), dense(L.up), dense(L.down)
    g_ref = TF.linear(T(r["a"]), T(Wg)).numpy()
    u_ref = TF.linear(T(r["a"]), T(Wu)).numpy()
    assert np.allclose(r["g"], g_ref, rtol=0, atol=1e-12 * r["ag"].max())
    assert np.allclose(r["u"], u_ref, rtol=0, atol=1e-12 * r["au"].max())
    s_pre = TF.silu(T(r["g"])).numpy() * r["u"]
    assert np.array_equal(r["s"], chain.bf16_round(s_pre))
    # swapping the roles of gate and up gives something else
    assert not np.array_equal(chain.bf16_round(TF.silu(T(r["u"])).numpy() * r["g"]), r["s"])

    # the down product of s, added to the residual
    y_ref = TF.linear(T(r["s"]), T(Wd)).numpy()
    assert np.allclose(r["y"], y_ref, rtol=0, atol=1e-12 * r["ay"].max())
    assert np.allclose(r["h"], h + y_ref, rtol=0, atol=1e-12 * (r["ay"].max() + np.abs(h).max()))


def test_mlp_layer_invariants():
    D, F, N = 64, 32, 2
    L = inputs.mlp_layer_inputs(D, F, 21)
    h = inputs.residual_inputs(N, D, 22).astype(np.float64)
    args = (as_tuple(L.gate), as_tuple(L.up), as_tuple(L.down), L.gamma)
    # without eps the normalization removes a positive scale of h (powers of
    # two keep every value exact)
    r1 = chain.mlp_layer(h, *args, 0.0)
    r4 = chain.mlp_layer(4.0 * h, *args, 0.0)
    assert np.array_equal(r1["a"], r4["a"]) and np.array_equal(r1["s"], r4["s"])
    assert np.array_equal(r4["y"], r1["y"]) and np.array_equal(r4["h"], 4.0 * h + r1["y"])
    # a column's result does not depend on the other columns
    rc = chain.mlp_layer(h[1:2], *args, 0.0)
    assert np.array_equal(rc["h"][0], r1["h"][1])
    # all-zero down codes: the residual passes through unchanged
    down0 = (np.zeros_like(L.down.codes), L.down.scales, L.down.g)
    assert np.array_equal(chain.mlp_layer(h, args[0], args[1], down0, L.gamma, 1e-6)["h"], h)
    # gamma = 0: nothing reaches the products
    r0 = chain.mlp_layer(h, *args[:3], np.zeros(D, np.uint16), 1e-6)
    assert not r0["a"].any() and not r0["s"].any() and np.array_equal(r0["h"], h)


def test_mlp_chain_is_layers_in_order():
    D, F, N = 32, 32, 2
    Ls = [inputs.mlp_layer_inputs(D, F, 30 + i) for i in range(3)]
    h = inputs.residual_inputs(N, D, 33).astype(np.float64)
    layers = [(as_tuple(L.gate), as_tuple(L.up), as_tuple(L.down), L.gamma) for L in Ls]
    out = chain.mlp_chain(h, layers, 1e-6)
    # layers do not commute: reversing them changes the result
    assert not np.allclose(out, chain.mlp_chain(h, layers[::-1], 1e-6))
    # each layer's output is the next one's input
    mid = chain.mlp_chain(h, layers[:2], 1e-6)
    assert np.array_equal(chain.mlp_chain(mid, layers[2:], 1e-6), out)
