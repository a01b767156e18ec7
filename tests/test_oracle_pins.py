"""Pins of the CPU oracle against facts fixed outside it.

Nothing here compares the oracle with itself.  The expected values come from
the format specifications (fixtures under tests/golden/, each citing its
source), from torch's own float8/bfloat16 casts (an independent library),
from closed forms, from invariants of a bilinear product, and from exact
rational arithmetic on tiny inputs.  Each test is chosen so that a plausible
slip in the oracle -- a swapped nibble, a wrong block index, a dropped scale,
a transposed operand, a wrong sign -- fails at least one of them.

The pages this build follows (crit-hub "mtp7-device-confidence", sections
"Design" and "Checks") print no product values, so parity with the pages
themselves is not pinnable; the pins are the format definitions and the
mathematics of y = W x.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from fp8_weight_streaming_amd import inputs
from golden_util import e2m1_table, read_table

E2M1 = e2m1_table()


def torch_e4m3(byte):
    """E4M3 value from torch's float8_e4m3fn cast (independent of the oracle)."""
    t = torch.tensor([byte], dtype=torch.uint8).view(torch.float8_e4m3fn)
    return float(t.to(torch.float64)[0])


def frac_bf16(bits):
    return Fraction(float(inputs.bf16_to_f32(np.array([bits], np.uint16))[0]))


def ref_w_nvfp4(codes, scales, g):
    """Exact rational weights from the golden E2M1 table and torch's E4M3."""
    M, half = codes.shape
    K = 2 * half
    e4 = {b: Fraction(torch_e4m3(b)) for b in range(256) if (b & 0x7F) != 0x7F}
    W = [[None] * K for _ in range(M)]
    for m in range(M):
        for k in range(K):
            byte = int(codes[m, k // 2])
            code = byte & 0xF if k % 2 == 0 else byte >> 4
            W[m][k] = E2M1[code] * e4[int(scales[m, k // 16])] * Fraction(float(np.float32(g)))
    return W


def exact_product(W, x):
    N, K = x.shape
    M = len(W)
    X = [[frac_bf16(int(x[n, k])) for k in range(K)] for n in range(N)]
    y = [[sum(W[m][k] * X[n][k] for k in range(K)) for m in range(M)] for n in range(N)]
    a = [[sum(abs(W[m][k] * X[n][k]) for k in range(K)) for m in range(M)] for n in range(N)]
    return y, a


ONE_BF16 = 0x3F80


# ---- P1 / P2: element decoders -----------------------------------------

def test_e2m1_all_codes_match_spec_table():
    for code, want in E2M1.items():
        got = oracle.e2m1(code)
        assert Fraction(got) == want, code
        assert math.copysign(1.0, got) == (-1.0 if code & 8 else 1.0)  # -0 keeps its sign


def test_e4m3_all_bytes_match_torch():
    for b in range(256):
        want = torch_e4m3(b)
        got = oracle.e4m3(b)
        if math.isnan(want):
            assert math.isnan(got), hex(b)
        else:
            assert got == want and math.copysign(1, got) == math.copysign(1, want), hex(b)


def test_e4m3_spec_boundary_values():
    for b, v in read_table("e4m3_special.txt"):
        got = oracle.e4m3(b)
        if v == "nan":
            assert math.isnan(got)
        else:
            assert got == float(v) and math.copysign(1, got) == math.copysign(1, float(v)), hex(b)


def test_bf16_decode_matches_torch():
    rng = np.random.default_rng(5)
    bits = np.concatenate([rng.integers(0, 65536, 2000), [0, 0x8000, 0x3F80, 0x7F7F, 0x0001, 0x8001]])
    bits = bits[(bits & 0x7F80) != 0x7F80].astype(np.uint16)  # finite patterns
    want = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([oracle.bf16(int(b)) for b in bits])
    assert np.array_equal(got, want)


# ---- P3: every code x selected scales, closed form ----------------------

@pytest.mark.parametrize("g", [1.0, 0.02])
def test_codes_times_scales_closed_form(g):
    scale_bytes = [0x01, 0x07, 0x08, 0x38, 0x39, 0x55, 0x7E]
    K = 32
    rows = [(c, s) for c in range(16) for s in scale_bytes]
    M = len(rows)
    codes = np.zeros((M, K // 2), np.uint8)
    scales = np.zeros((M, K // 16), np.uint8)
    for m, (c, s) in enumerate(rows):
        codes[m, :] = c | (c << 4)
        scales[m, :] = s
    x = np.full((1, K), ONE_BF16, np.uint16)
    y, a = oracle.gemm_nvfp4(codes, scales, g, x)
    g32 = Fraction(float(np.float32(g)))
    for m, (c, s) in enumerate(rows):
        want = 32 * E2M1[c] * Fraction(torch_e4m3(s)) * g32
        assert Fraction(y[0, m]) == want, (c, s)
        assert Fraction(a[0, m]) == abs(want)


# ---- P4: one-hot columns pick single weights (nibble order, block index) --

def test_one_hot_columns_select_weights():
    M, K, N = 5, 96, 7
    d = inputs.nvfp4_inputs(M, K, 1, seed=11)
    ks = [0, 1, 15, 16, 17, 63, 95]
    x = np.zeros((N, K), np.uint16)
    for n, k in enumerate(ks):
        x[n, k] = ONE_BF16
    g = 0.02
    y, a = oracle.gemm_nvfp4(d.codes, d.scales, g, x)
    W = ref_w_nvfp4(d.codes, d.scales, g)
    for n, k in enumerate(ks):
        for m in range(M):
            assert Fraction(y[n, m]) == W[m][k], (n, m, k)
            assert Fraction(a[n, m]) == abs(W[m][k])


# ---- P5: identity -------------------------------------------------------

def test_identity_weights_reproduce_x():
    K = 32
    codes = np.zeros((K, K // 2), np.uint8)
    for m in range(K):
        codes[m, m // 2] = 0x2 << (4 * (m % 2))  # code 0x2 = 1.0 on the diagonal
    scales = np.full((K, K // 16), 0x38, np.uint8)  # 1.0
    d = inputs.nvfp4_inputs(1, K, 3, seed=3)
    y, _ = oracle.gemm_nvfp4(codes, scales, 1.0, d.x)
    assert np.array_equal(y, inputs.bf16_to_f32(d.x).astype(np.float64))


# ---- P6: brute force against exact rational sums ------------------------

@pytest.mark.parametrize("seed", [21, 22])
def test_brute_force_exact_sums_k32(seed):
    M, K, N = 6, 32, 3
    d = inputs.nvfp4_inputs(M, K, N, seed=seed, g=0.02)
    d.scales[0, 0] = 0x03  # subnormal scale
    d.scales[1, 1] = 0x00  # zero scale
    y, a = oracle.gemm_nvfp4(d.codes, d.scales, d.g, d.x)
    W = ref_w_nvfp4(d.codes, d.scales, d.g)
    ye, ae = exact_product(W, d.x)
    for n in range(N):
        for m in range(M):
            bound = K * Fraction(2) ** -53 * ae[n][m]
            assert abs(Fraction(y[n, m]) - ye[n][m]) <= bound, (n, m)
            assert abs(Fraction(a[n, m]) - ae[n][m]) <= bound, (n, m)


def test_row_subset_equals_full_rows():
    d = inputs.nvfp4_inputs(40, 160, 4, seed=9, g=0.02)
    y, a = oracle.gemm_nvfp4(d.codes, d.scales, d.g, d.x)
    rows = np.array([39, 0, 17, 17, 5])
    ys, as_ = oracle.gemm_nvfp4(d.codes, d.scales, d.g, d.x, rows=rows)
    assert np.array_equal(ys, y[:, rows]) and np.array_equal(as_, a[:, rows])


# ---- P7: invariants of the bilinear product ------------------------------

def test_invariants_nvfp4():
    M, K, N = 24, 256, 4
    d = inputs.nvfp4_inputs(M, K, N, seed=31, g=0.02)
    y, a = oracle.gemm_nvfp4(d.codes, d.scales, d.g, d.x)
    # flipping every code's sign bit negates y
    y_neg, a_neg = oracle.gemm_nvfp4(d.codes ^ np.uint8(0x88), d.scales, d.g, d.x)
    assert np.array_equal(y_neg, -y) and np.array_equal(a_neg, a)
    # doubling g doubles y
    y2, _ = oracle.gemm_nvfp4(d.codes, d.scales, 2 * d.g, d.x)
    assert np.array_equal(y2, 2 * y)
    # swapping two activation columns swaps the matching output rows
    xs = d.x[[2, 1, 0, 3]]
    ysw, _ = oracle.gemm_nvfp4(d.codes, d.scales, d.g, xs)
    assert np.array_equal(ysw, y[[2, 1, 0, 3]])
    # scaling x by 2^3 (add 3 to every BF16 exponent) scales y by 8
    nz = (d.x & 0x7F80) != 0
    x8 = d.x.copy()
    x8[nz] = x8[nz] + np.uint16(3 << 7)
    y8, _ = oracle.gemm_nvfp4(d.codes, d.scales, d.g, x8)
    assert np.array_equal(y8, 8 * y)
    # the sum of two weight matrices that split the codes is the sum of products
    lo = d.codes & np.uint8(0x0F)
    hi = d.codes & np.uint8(0xF0)
    y_lo, _ = oracle.gemm_nvfp4(lo, d.scales, d.g, d.x)
    y_hi, _ = oracle.gemm_nvfp4(hi, d.scales, d.g, d.x)
    assert np.allclose(y_lo + y_hi, y, rtol=0, atol=1e-12 * np.abs(a).max())


def test_scale_block_applies_to_sixteen_k():
    # one scale block changed -> only the contribution of its 16 k changes
    M, K, N = 3, 64, 2
    d = inputs.nvfp4_inputs(M, K, N, seed=41)
    s2 = d.scales.copy()
    s2[:, 2] = 0x00  # zero the block covering k = 32..47
    y, _ = oracle.gemm_nvfp4(d.codes, d.scales, 1.0, d.x)
    y2, _ = oracle.gemm_nvfp4(d.codes, s2, 1.0, d.x)
    xm = d.x.copy()
    xm[:, 32:48] = 0
    y3, _ = oracle.gemm_nvfp4(d.codes, d.scales, 1.0, xm)
    assert np.allclose(y2, y3, rtol=0, atol=1e-12)
    assert not np.allclose(y, y2)


# ---- P8: the FP8-row path -------------------------------------------------

def test_fp8row_one_hot_and_row_scale():
    M, K, N = 4, 48, 3
    rng = np.random.default_rng(1)
    w = rng.integers(0, 256, size=(M, K), dtype=np.uint8)
    w[(w & 0x7F) == 0x7F] = 0x38  # keep NaN encodings out of this one
    r = np.array([1.0, 0.5, 3.0, 0.01], np.float32)
    ks = [0, 17, 47]
    x = np.zeros((N, K), np.uint16)
    for n, k in enumerate(ks):
        x[n, k] = ONE_BF16
    y, a = oracle.gemm_fp8row(w, r, x)
    for n, k in enumerate(ks):
        for m in range(M):
            want = Fraction(torch_e4m3(int(w[m, k]))) * Fraction(float(r[m]))
            assert Fraction(y[n, m]) == want and Fraction(a[n, m]) == abs(want)


def test_fp8row_brute_force_and_invariants():
    M, K, N = 5, 32, 2
    d = inputs.fp8row_inputs(M, K, N, seed=7)
    y, a = oracle.gemm_fp8row(d.w, d.row_scale, d.x)
    X = [[frac_bf16(int(d.x[n, k])) for k in range(K)] for n in range(N)]
    for n in range(N):
        for m in range(M):
            terms = [Fraction(torch_e4m3(int(d.w[m, k]))) * Fraction(float(d.row_scale[m])) * X[n][k]
                     for k in range(K)]
            ye, ae = sum(terms), sum(abs(t) for t in terms)
            bound = K * Fraction(2) ** -53 * ae
            assert abs(Fraction(y[n, m]) - ye) <= bound and abs(Fraction(a[n, m]) - ae) <= bound
    y_neg, _ = oracle.gemm_fp8row(d.w ^ np.uint8(0x80), d.row_scale, d.x)
    assert np.array_equal(y_neg, -y)
    y2, _ = oracle.gemm_fp8row(d.w, 2 * d.row_scale, d.x)
    assert np.array_equal(y2, 2 * y)
    ysw, _ = oracle.gemm_fp8row(d.w, d.row_scale, d.x[::-1])
    assert np.array_equal(ysw, y[::-1])


def test_nan_scale_propagates_and_zero_scale_silences():
    K = 32
    codes = np.full((3, K // 2), 0x22, np.uint8)
    scales = np.array([[0x38, 0x38], [0x7F, 0x38], [0x00, 0x00]], np.uint8)
    x = np.full((1, K), ONE_BF16, np.uint16)
    y, _ = oracle.gemm_nvfp4(codes, scales, 1.0, x)
    assert y[0, 0] == 32.0 and math.isnan(y[0, 1]) and y[0, 2] == 0.0
