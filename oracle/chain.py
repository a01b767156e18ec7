"""A chained MLP verify pass -- TEST INFRASTRUCTURE ONLY (same rule as the
rest of ``oracle``: only tests, the smoke check and the CPU-baseline leg of
the benchmark may import it).

What the pages fix: the crit-hub engine card "mtp7-device-confidence"
(section "Limits") puts its short-prompt latency on the many small kernels
each layer launches, and (section "Design", row "Decode") runs a decode
round as one device graph.  They give no layer equations.  Reading taken
here -- a dense MLP block applied to the N verify columns, with an FP32
residual stream h [N][D]:

    r[n]   = 1 / sqrt(mean_k h[n][k]^2 + eps)
    a      = BF16(h * r * gamma)                     gamma: BF16 [D]
    g, u   = a . Wg^T,  a . Wu^T                     NVFP4 [F][D] each
    s      = BF16(silu(g) * u),  silu(v) = v / (1 + exp(-v))
    h'     = h + s . Wd^T                            NVFP4 [D][F]

Everything is FP64 except the two BF16 roundings the definition makes (a
and s are the BF16 inputs of the next products): round to nearest, ties
to even, once, from the FP64 value.  eps is taken as the FP32 number the
library receives.

Pins: tests/test_chain_pins.py (torch's float32 -> bfloat16 cast, torch's
float64 rms_norm / silu / linear on decoded weights, scale invariance and
zero-weight special cases).
"""
from __future__ import annotations

import numpy as np

import oracle


def bf16_round(v) -> np.ndarray:
    """FP64 -> nearest BF16 value, ties to even, as float64 (one rounding).

    BF16 keeps 8 significant bits and FP32's exponent range: normal values
    are quantized to 2^(e-8) for v = m 2^e, 0.5 <= |m| < 1, values below
    2^-126 to the subnormal step 2^-133; magnitudes that round to 2^128 or
    more become infinite.  NaN stays NaN, +-0 and +-inf stay."""
    v = np.asarray(v, dtype=np.float64)
    out = v.copy()
    fin = np.isfinite(v) & (v != 0.0)
    x = v[fin]
    _, e = np.frexp(x)
    q = np.maximum(e - 8, -133)
    r = np.ldexp(np.rint(np.ldexp(x, -q)), q)   # both scalings are exact
    big = np.abs(r) >= 2.0 ** 128
    r[big] = np.copysign(np.inf, r[big])
    out[fin] = r
    return out


def bf16_value(bits) -> np.ndarray:
    """BF16 bit patterns -> their values (float64)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def bf16_bits(v) -> np.ndarray:
    """Bit patterns of values that are BF16 numbers already (exact)."""
    f = np.asarray(v, dtype=np.float64).astype(np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def silu(v) -> np.ndarray:
    v = np.asarray(v, dtype=np.float64)
    with np.errstate(over="ignore"):
        return v / (1.0 + np.exp(-v))


def rmsnorm(h, gamma_bits, eps: float) -> np.ndarray:
    """h * r * gamma before rounding (FP64), r per column as above."""
    h = np.asarray(h, dtype=np.float64)
    e = float(np.float32(eps))
    r = 1.0 / np.sqrt((h * h).mean(axis=1, keepdims=True) + e)
    return h * r * bf16_value(gamma_bits)[None, :]


def normalize(h, gamma_bits, eps: float) -> np.ndarray:
    """a = BF16(h * r * gamma): the BF16 input of the gate/up products."""
    return bf16_round(rmsnorm(h, gamma_bits, eps))


def mlp_layer(h, gate, up, down, gamma_bits, eps: float) -> dict:
    """One layer on columns h [N][D] (float64 or float32 values).

    gate, up, down: (codes uint8 [R][C/2], scales uint8 [R][C/16], g float)
    in the plain NVFP4 layout.  Returns float64 arrays: a (BF16 values),
    g, u (FP64 products), ag, au (their sums of |w x|, the scale of a
    product's rounding error), s (BF16 values), y (s . Wd^T), ay, and the
    new residual h."""
    h = np.asarray(h, dtype=np.float64)
    a = normalize(h, gamma_bits, eps)
    xa = bf16_bits(a)
    g, ag = oracle.gemm_nvfp4(gate[0], gate[1], gate[2], xa)
    u, au = oracle.gemm_nvfp4(up[0], up[1], up[2], xa)
    s = bf16_round(silu(g) * u)
    y, ay = oracle.gemm_nvfp4(down[0], down[1], down[2], bf16_bits(s))
    return {"a": a, "g": g, "u": u, "ag": ag, "au": au, "s": s, "y": y, "ay": ay, "h": h + y}


def mlp_chain(h, layers, eps: float) -> np.ndarray:
    """Layers applied in order; layers = [(gate, up, down, gamma_bits)]."""
    h = np.asarray(h, dtype=np.float64)
    for gate, up, down, gamma in layers:
        h = mlp_layer(h, gate, up, down, gamma, eps)["h"]
    return h
