"""Seeded synthetic inputs for the verify-pass product.

This module only *draws* inputs: raw weight codes, block scales, row scales
and BF16 activations, as host numpy arrays.  It holds none of the product's
arithmetic (no decoding, no multiply-accumulate); both the HIP path and the
CPU oracle consume what it returns.  Encoding to E4M3 and BF16 uses torch's
round-to-nearest-even casts (``torch.float8_e4m3fn``, ``torch.bfloat16``).

There is no checkpoint here: the weights the crit-hub engine card
"mtp7-device-confidence" streams (section "Model") are replaced by random
arrays with the block structure of their formats and the shapes of a dense
64-layer target (section "Measured": a verify pass reads every weight once).

Recipe (every draw from ``numpy.random.Generator(PCG64(seed))``, in the order
listed):

NVFP4 matrix (M x K):
  codes   uint8 [M, K/2]   uniform bytes, so both nibbles are uniform over
                           all 16 E2M1 codes
  scales  uint8 [M, K/16]  E4M3 round-to-nearest-even of 2**u,
                           u ~ U[-4, 2] (continuous, drawn in float64,
                           2**u rounded to float32 before the E4M3 cast)
  g       float32          per-tensor multiplier, set by the workload
  x       uint16 [N, K]    BF16 round-to-nearest-even of float32(z * xs),
                           z ~ N(0, 1), xs set by the workload

Row-scaled FP8-E4M3 matrix (M x K):
  wb      BF16 of float32(0.02 * z), z ~ N(0, 1), shape [M, K]
  r[m]    float32(max_k |wb[m, k]| / 448)   (0 for an all-zero row)
  w       uint8 [M, K] E4M3 round-to-nearest-even of float32(wb / r)
          (0 where r == 0); |wb / r| <= 448 so nothing saturates
  x       as above with xs = 1
  The BF16 weights wb are dropped; only w and r are returned.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List

import numpy as np
import torch


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(int(seed)))


def to_e4m3(values: np.ndarray) -> np.ndarray:
    """float32 array -> E4M3 (FN) bytes, round-to-nearest-even (torch cast)."""
    t = torch.from_numpy(np.ascontiguousarray(values, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def to_bf16(values: np.ndarray) -> np.ndarray:
    """float32 array -> BF16 bit patterns (uint16), round-to-nearest-even."""
    t = torch.from_numpy(np.ascontiguousarray(values, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """BF16 bit patterns -> float32 (exact widening)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


@dataclass
class NVFP4Inputs:
    codes: np.ndarray   # uint8 [M, K/2]
    scales: np.ndarray  # uint8 [M, K/16]
    g: float            # float32 value
    x: np.ndarray       # uint16 [N, K]

    @property
    def M(self) -> int:
        return self.codes.shape[0]

    @property
    def K(self) -> int:
        return 2 * self.codes.shape[1]


@dataclass
class FP8RowInputs:
    w: np.ndarray          # uint8 [M, K]
    row_scale: np.ndarray  # float32 [M]
    x: np.ndarray          # uint16 [N, K]

    @property
    def M(self) -> int:
        return self.w.shape[0]

    @property
    def K(self) -> int:
        return self.w.shape[1]


def nvfp4_inputs(M: int, K: int, N: int, seed: int, g: float = 1.0,
                 x_scale: float = 1.0) -> NVFP4Inputs:
    """Draw one NVFP4 matrix and N BF16 activation columns."""
    if K % 32:
        raise ValueError("NVFP4 K must be a multiple of 32")
    rng = _rng(seed)
    codes = rng.integers(0, 256, size=(M, K // 2), dtype=np.uint8)
    u = rng.uniform(-4.0, 2.0, size=(M, K // 16))
    scales = to_e4m3(np.exp2(u).astype(np.float32))
    z = rng.standard_normal(size=(N, K), dtype=np.float32)
    x = to_bf16(z * np.float32(x_scale))
    return NVFP4Inputs(codes=codes, scales=scales, g=float(np.float32(g)), x=x)


def fp8row_inputs(M: int, K: int, N: int, seed: int) -> FP8RowInputs:
    """Draw one row-scaled FP8-E4M3 matrix and N BF16 activation columns."""
    if K % 16:
        raise ValueError("FP8-row K must be a multiple of 16")
    rng = _rng(seed)
    wb = bf16_to_f32(to_bf16(rng.standard_normal(size=(M, K), dtype=np.float32) * np.float32(0.02)))
    rowmax = np.abs(wb).max(axis=1) if K else np.zeros(M, np.float32)
    r = (rowmax / np.float32(448.0)).astype(np.float32)
    safe = np.where(r > 0, r, np.float32(1.0)).astype(np.float32)
    q = (wb / safe[:, None]).astype(np.float32)
    q[r == 0] = 0.0
    w = to_e4m3(q)
    z = rng.standard_normal(size=(N, K), dtype=np.float32)
    x = to_bf16(z)
    return FP8RowInputs(w=w, row_scale=r, x=x)


# ---- hashed rows: matrices too large to draw ------------------------------
# The largest matrices the tiled layouts address hold just under 2**32 bytes;
# drawing all their weights from PCG64 on the host takes tens of GB of
# temporaries.  These functions give any chosen rows of such a matrix
# instead, from a closed-form hash of (seed, row, column): a test builds the
# matrix on the device chunk by chunk and hands the oracle only the rows it
# checks.  Every row differs from every other, so a tile read from the wrong
# place shows.  Byte (m, j) is the top byte of h(m) * h'(j) (mod 2**32), with
# h and h' xorshift-multiply mixes of the row and column indices and h'
# forced odd: two rows a, b then differ by (h(a) - h(b)) * h'(j) in column
# j, which reaches the top byte for nearly every j.

def _mix32(a: np.ndarray, seed: int) -> np.ndarray:
    """xorshift-multiply mix of uint32 values (a fixed bijection per seed)."""
    a = (np.asarray(a, dtype=np.uint64) ^ np.uint64(seed & 0xFFFFFFFF)) & np.uint64(0xFFFFFFFF)
    for mul in (0x9E3779B1, 0x85EBCA6B, 0xC2B2AE35):
        a = (a ^ (a >> np.uint64(15))) * np.uint64(mul) & np.uint64(0xFFFFFFFF)
    return (a ^ (a >> np.uint64(16))).astype(np.uint32)


def _hashed_bytes(rows: np.ndarray, cols: int, seed: int) -> np.ndarray:
    """uint8 [len(rows), cols]: the top byte of h(row) * h'(col) mod 2**32."""
    hr = _mix32(np.asarray(rows, dtype=np.uint64), seed)[:, None]
    hc = (_mix32(np.arange(cols, dtype=np.uint64), seed ^ 0x5A5A5A5A) | np.uint32(1))[None, :]
    return ((hr * hc) >> np.uint32(24)).astype(np.uint8)


# E4M3 block scales of the hashed matrices: 2**e and 1.5 * 2**e, e in [-4, 3]
_HASHED_SCALES = np.array([((e + 7) << 3) | m for e in range(-4, 4) for m in (0, 4)], dtype=np.uint8)


def hashed_nvfp4_rows(rows: np.ndarray, K: int, seed: int):
    """Rows `rows` of a hashed NVFP4 matrix with K columns: (codes uint8
    [len(rows), K/2], uniform-looking bytes; scales uint8 [len(rows), K/16]
    from the 16 table values above)."""
    if K % 32:
        raise ValueError("NVFP4 K must be a multiple of 32")
    codes = _hashed_bytes(rows, K // 2, seed)
    scales = _HASHED_SCALES[_hashed_bytes(rows, K // 16, seed + 1) >> 4]
    return codes, scales


def hashed_fp8_rows(rows: np.ndarray, K: int, seed: int):
    """Rows `rows` of a hashed row-scaled FP8-E4M3 matrix: (w uint8
    [len(rows), K], bytes with the lowest exponent bit cleared, so no NaN
    code; row_scale float32 [len(rows)], 2**-10 * (1 + j / 8), j in 0..7)."""
    w = _hashed_bytes(rows, K, seed) & np.uint8(0xF7)
    j = _mix32(np.asarray(rows, dtype=np.uint64), seed + 2) >> np.uint32(29)
    r = (np.float32(2.0 ** -10) * (np.float32(1.0) + j.astype(np.float32) / np.float32(8.0))).astype(np.float32)
    return w, r


# ---- the five workloads --------------------------------------------------

@dataclass
class MatrixSpec:
    name: str
    M: int
    K: int


@dataclass
class Workload:
    index: int
    name: str
    fmt: str                 # "nvfp4" or "fp8row"
    N: int                   # columns (for the verify pass: the largest N)
    g: float = 1.0
    x_scale: float = 1.0
    matrices: List[MatrixSpec] = field(default_factory=list)
    n_cycle: List[int] = field(default_factory=list)

    def seed(self, matrix_index: int) -> int:
        return 1000 * self.index + matrix_index


VERIFY_LAYER = [MatrixSpec("qkv", 7168, 5120), MatrixSpec("o", 5120, 6144),
                MatrixSpec("gate_up", 34816, 5120), MatrixSpec("down", 5120, 17408)]


def workload(index: int, layers: int = 64) -> Workload:
    """The five synthetic workloads (index 0-4)."""
    g02 = float(np.float32(0.02))
    if index == 0:
        return Workload(0, "nvfp4 gemv 1024x1024 N=1", "nvfp4", 1, 1.0, 1.0,
                        [MatrixSpec("w", 1024, 1024)])
    if index == 1:
        return Workload(1, "nvfp4 decode gemv up-proj 17408x5120 N=1", "nvfp4", 1, g02, 0.5,
                        [MatrixSpec("w", 17408, 5120)])
    if index == 2:
        return Workload(2, "nvfp4 verify gemm down-proj 5120x17408 N=8", "nvfp4", 8, g02, 1.0,
                        [MatrixSpec("w", 5120, 17408)])
    if index == 3:
        mats = [MatrixSpec("L%d.%s" % (l, s.name), s.M, s.K) for l in range(layers) for s in VERIFY_LAYER]
        return Workload(3, "nvfp4 dense verify pass %d layers x {qkv 7168x5120, o 5120x6144, "
                        "gate+up 34816x5120, down 5120x17408}, N cycled 2,4,8" % layers,
                        "nvfp4", 8, g02, 1.0, mats, [2, 4, 8])
    if index == 4:
        return Workload(4, "fp8-row output head 151936x5120 N=8", "fp8row", 8, 1.0, 1.0,
                        [MatrixSpec("head", 151936, 5120)])
    raise ValueError("workload index must be 0-4")


def workload_inputs(wl: Workload, matrix_index: int = 0):
    """Inputs of one matrix of a workload (N = the workload's largest N)."""
    spec = wl.matrices[matrix_index]
    if wl.fmt == "nvfp4":
        return nvfp4_inputs(spec.M, spec.K, wl.N, wl.seed(matrix_index), wl.g, wl.x_scale)
    return fp8row_inputs(spec.M, spec.K, wl.N, wl.seed(matrix_index))


# ---- chained MLP layers --------------------------------------------------

# rms of the stored NVFP4 weight values drawn by nvfp4_inputs with g = 1:
# E2M1 codes uniform over all 16 (mean square 68.5 / 8) times block scales
# 2^U(-4, 2) (mean square (16 - 4^-4) / (6 ln 4)).
NVFP4_DRAW_RMS = float(np.sqrt(68.5 / 8 * (16.0 - 4.0 ** -4) / (6.0 * np.log(4.0))))


@dataclass
class MlpLayerInputs:
    gate: NVFP4Inputs   # [F][D]  (x unused)
    up: NVFP4Inputs     # [F][D]
    down: NVFP4Inputs   # [D][F]
    gamma: np.ndarray   # uint16 [D] BF16 norm weights


def mlp_layer_inputs(D: int, F: int, seed: int, down_gain: float = 0.25, up_gain: float = 1.0) -> MlpLayerInputs:
    """Weights of one MLP layer.  Tensor scales put the gate/up outputs near
    unit size for unit-size normalized inputs, and scale each layer's
    addition to the residual by about down_gain, so that a stack of many
    layers stays in range."""
    g_gu = float(np.float32(1.0 / (NVFP4_DRAW_RMS * np.sqrt(D))))
    g_d = float(np.float32(down_gain / (NVFP4_DRAW_RMS * np.sqrt(F))))
    gate = nvfp4_inputs(F, D, 1, 4 * seed + 0, g_gu)
    up = nvfp4_inputs(F, D, 1, 4 * seed + 1, float(np.float32(g_gu * up_gain)))
    down = nvfp4_inputs(D, F, 1, 4 * seed + 2, g_d)
    rng = _rng(4 * seed + 3)
    gamma = to_bf16((1.0 + 0.2 * rng.standard_normal(D)).astype(np.float32))
    return MlpLayerInputs(gate, up, down, gamma)


def residual_inputs(N: int, D: int, seed: int) -> np.ndarray:
    """FP32 residual-stream columns [N][D]."""
    return _rng(seed).standard_normal(size=(N, D), dtype=np.float32)
