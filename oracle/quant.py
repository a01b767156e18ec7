"""Round-to-nearest quantizers -- TEST INFRASTRUCTURE ONLY (same rule as
the rest of ``oracle``).

What the pages say: the crit landing page, section on Models, produces
transformed weights by post-training quantization to FP8 or NVFP4 with
round-to-nearest; the Gemma case study there re-encodes BF16 projections
and the output head to FP8 at load; the crit-hub engine card
"mtp7-device-confidence", section "Model", re-encodes its draft layer as
row-scaled FP8 and its output head as NVFP4.  They give no formula.
Reading, written out here:

FP8-row, per row m of BF16 weights w:
    r[m] = fp32(max_k |w[m][k]| / 448)
    q[m][k] = E4M3(fp32(w[m][k] / r[m]))      (0 for a zero row, r = 0)

NVFP4, with a given FP32 tensor scale g (> 0), per block of 16 k:
    s = E4M3(fp32(max |w| over the block / fp32(6 * g)))
    d = fp32(e4m3(s) * g)
    code_k = E2M1(fp32(w_k / d))               (0 for every k when d = 0)

E4M3(v) and E2M1(v) are round-to-nearest, ties to the even code, onto the
finite values of the format (values past the largest saturate to it); the
sign bit is the sign of v, so a negative value that rounds to zero gives
the negative zero code.  Here they are written as a search for the nearest
entry of the decoded code table -- the plain definition -- not as bit
arithmetic.  Inputs are finite.
"""
from __future__ import annotations

import numpy as np

from oracle import bf16, e2m1, e4m3


def _table(decode, codes):
    vals = np.array([decode(c) for c in codes], dtype=np.float64)
    return np.asarray(codes), vals


_E4M3_MAG = _table(e4m3, list(range(0x7F)))     # +0 .. 448 (0x7F is NaN)
_E2M1_MAG = _table(e2m1, list(range(8)))        # +0 .. 6


def _nearest(a: np.ndarray, table) -> np.ndarray:
    """Code of the table value nearest each |a|; ties go to the even code."""
    codes, vals = table
    d = np.abs(a[..., None] - vals)              # distance to every magnitude
    best = d.min(axis=-1, keepdims=True)
    cand = d == best                             # one or two candidates
    even = cand & ((codes & 1) == 0)
    pick = np.where(even.any(axis=-1, keepdims=True), even, cand)
    return codes[np.argmax(pick, axis=-1)]


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    v = np.asarray(v, dtype=np.float32)
    mag = _nearest(np.abs(v).astype(np.float64), _E4M3_MAG).astype(np.uint8)
    return mag | (np.signbit(v).astype(np.uint8) << 7)


def e2m1_encode(v: np.ndarray) -> np.ndarray:
    v = np.asarray(v, dtype=np.float32)
    mag = _nearest(np.abs(v).astype(np.float64), _E2M1_MAG).astype(np.uint8)
    return mag | (np.signbit(v).astype(np.uint8) << 3)


def _bf16_to_f32(w: np.ndarray) -> np.ndarray:
    return (np.asarray(w, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def quantize_fp8row(w_bf16: np.ndarray):
    """(q uint8 [M][K], r float32 [M]) from BF16 bits [M][K]."""
    w = _bf16_to_f32(w_bf16)
    rowmax = np.abs(w).max(axis=1)
    r = (rowmax / np.float32(448.0)).astype(np.float32)
    q = np.zeros(w.shape, dtype=np.uint8)
    for m in range(w.shape[0]):
        if r[m] > 0:
            q[m] = e4m3_encode((w[m] / r[m]).astype(np.float32))
    return q, r


def quantize_nvfp4(w_bf16: np.ndarray, g: float):
    """(codes uint8 [M][K/2], scales uint8 [M][K/16]) from BF16 bits [M][K]."""
    w = _bf16_to_f32(w_bf16)
    M, K = w.shape
    g = np.float32(g)
    six_g = np.float32(np.float32(6.0) * g)
    codes = np.zeros((M, K // 2), dtype=np.uint8)
    scales = np.zeros((M, K // 16), dtype=np.uint8)
    for m in range(M):
        blocks = w[m].reshape(K // 16, 16)
        amax = np.abs(blocks).max(axis=1)
        s = e4m3_encode((amax / six_g).astype(np.float32))
        sd = np.array([e4m3(int(c)) for c in s], dtype=np.float32)
        d = (sd * g).astype(np.float32)
        c16 = np.zeros((K // 16, 16), dtype=np.uint8)
        for b in np.flatnonzero(d > 0):
            c16[b] = e2m1_encode((blocks[b] / d[b]).astype(np.float32))
        flat = c16.reshape(K)
        codes[m] = flat[0::2] | (flat[1::2] << 4)
        scales[m] = s
    return codes, scales


__all__ = ["e4m3_encode", "e2m1_encode", "quantize_fp8row", "quantize_nvfp4", "bf16"]
