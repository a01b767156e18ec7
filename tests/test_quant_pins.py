"""Pins of the round-to-nearest quantizer oracle (CPU only): the encoders
invert the decoders on every code, send midpoints to the even code (the
OCP formats' round-to-nearest-even rule), agree with torch's E4M3 cast in
range; the FP8-row quantizer agrees with an independent torch formulation;
the NVFP4 quantizer reproduces exactly representable blocks and zero
blocks, and is invariant under scaling w and g by a power of two."""
import numpy as np
import pytest
import torch

from oracle import e2m1, e4m3
from oracle.quant import e2m1_encode, e4m3_encode, quantize_fp8row, quantize_nvfp4
from fp8_weight_streaming_amd.inputs import to_bf16


def test_encoders_invert_decoders():
    for c in list(range(0x7F)) + list(range(0x80, 0xFF)):
        assert e4m3_encode(np.array([e4m3(c)], np.float32))[0] == c, hex(c)
    for c in range(16):
        assert e2m1_encode(np.array([e2m1(c)], np.float32))[0] == c


def test_midpoints_go_to_the_even_code():
    # E2M1 magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6: each midpoint and the code it must take
    mids = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6}
    for v, c in mids.items():
        assert e2m1_encode(np.array([v], np.float32))[0] == c, v
        assert e2m1_encode(np.array([-v], np.float32))[0] == c | 8, -v
    assert e2m1_encode(np.array([6.5, 100.0, -7.0], np.float32)).tolist() == [7, 7, 15]   # saturate
    # E4M3: subnormal step 2^-9, normal 1.x with 3 mantissa bits, largest finite 448
    cases = {2.0 ** -10: 0x00, 3 * 2.0 ** -10: 0x02, 5 * 2.0 ** -10: 0x02, 1.0625: 0x38, 1.1875: 0x3A,
             15 * 2.0 ** -10: 0x08, 464.0: 0x7E, 1e9: 0x7E}
    for v, c in cases.items():
        assert e4m3_encode(np.array([v], np.float32))[0] == c, v
    assert e4m3_encode(np.array([-2.0 ** -12, -0.0], np.float32)).tolist() == [0x80, 0x80]


@pytest.mark.parametrize("seed", range(4))
def test_e4m3_encode_matches_torch_in_range(seed):
    rng = np.random.default_rng(seed)
    v = (rng.standard_normal(20000) * 10.0 ** rng.uniform(-4, 2.5, 20000)).astype(np.float32)
    v = v[np.abs(v) <= 448]
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(e4m3_encode(v), ref)


def test_fp8row_quantizer_matches_torch_formulation():
    rng = np.random.default_rng(5)
    w = to_bf16((rng.standard_normal((40, 96)) * 0.02).astype(np.float32))
    w[7] = 0  # a zero row
    q, r = quantize_fp8row(w)
    wf = torch.from_numpy((w.astype(np.uint32) << 16).view(np.float32))
    rt = (wf.abs().amax(dim=1) / 448.0).to(torch.float32)
    safe = torch.where(rt > 0, rt, torch.ones_like(rt))
    qt = (wf / safe[:, None]).to(torch.float8_e4m3fn).view(torch.uint8)
    qt[7] = 0
    assert np.array_equal(r, rt.numpy()) and np.array_equal(q, qt.numpy())
    assert r[7] == 0 and not q[7].any()


def _dequant(codes, scales, g):
    M = codes.shape[0]
    c = np.stack([codes & 15, codes >> 4], axis=2).reshape(M, -1)
    v = np.vectorize(e2m1)(c).astype(np.float64)
    s = np.vectorize(e4m3)(scales).astype(np.float64)
    return v * np.repeat(s, 16, axis=1) * g


def test_nvfp4_quantizer_reproduces_representable_blocks():
    rng = np.random.default_rng(6)
    g = np.float32(2.0 ** -7)
    M, K = 6, 64
    c = rng.integers(0, 16, (M, K)).astype(np.uint8)
    c[:, ::16] = 7            # every block holds a +6, so its scale is amax / 6 exactly
    s = rng.choice([0x30, 0x38, 0x3C, 0x44], (M, K // 16)).astype(np.uint8)
    wv = np.vectorize(e2m1)(c) * np.repeat(np.vectorize(e4m3)(s), 16, axis=1) * float(g)
    w = to_bf16(wv.astype(np.float32))
    assert np.array_equal((w.astype(np.uint32) << 16).view(np.float32), wv.astype(np.float32))  # exact in BF16
    codes, scales = quantize_nvfp4(w, g)
    assert np.array_equal(scales, s)
    assert np.array_equal(codes, (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8))


def test_nvfp4_quantizer_zero_blocks_and_scaling():
    rng = np.random.default_rng(7)
    g = np.float32(0.02 / 6)
    wf = (rng.standard_normal((8, 128)) * 0.02).astype(np.float32)
    wf[2, 16:32] = 0.0
    w = to_bf16(wf)
    codes, scales = quantize_nvfp4(w, g)
    assert scales[2, 1] == 0 and not (codes[2, 8:16]).any()
    # w * 2 and g * 2 give the same codes and scales
    w2 = to_bf16(((w.astype(np.uint32) << 16).view(np.float32) * 2).astype(np.float32))
    c2, s2 = quantize_nvfp4(w2, np.float32(g * 2))
    assert np.array_equal(c2, codes) and np.array_equal(s2, scales)
    # each dequantized value is the nearest representable one at its block scale
    deq = _dequant(codes, scales, float(g))
    wf64 = (w.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    sd = np.repeat(np.vectorize(e4m3)(scales).astype(np.float64), 16, axis=1) * float(g)
    grid = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])
    for m in range(8):
        for k in range(128):
            if sd[m, k] == 0:
                continue
            best = np.min(np.abs(np.abs(wf64[m, k]) / sd[m, k] - grid))
            assert abs(abs(wf64[m, k]) - abs(deq[m, k])) / sd[m, k] <= best + 1e-6
