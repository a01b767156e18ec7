"""The tiled NVFP4 layout's numpy statement is a permutation: every plain
byte appears once and the inverse restores it (CPU only)."""
import numpy as np
import pytest

from fp8_weight_streaming_amd import inputs
from tiled_ref import fp8_tile_ref, fp8_untile_ref, tile_ref, untile_ref


@pytest.mark.parametrize("M,K", [(1, 32), (16, 256), (17, 96), (40, 544), (33, 1056)])
def test_tile_ref_round_trip(M, K):
    d = inputs.nvfp4_inputs(M, K, 1, seed=M * 7 + K)
    t = tile_ref(d.codes, d.scales)
    assert t.size == -(-M // 16) * -(-K // 256) * 2304
    c, s = untile_ref(t, M, K)
    assert np.array_equal(c, d.codes) and np.array_equal(s, d.scales)


def test_tile_ref_places_bytes_as_documented():
    M, K = 20, 512
    codes = (np.arange(M * K // 2, dtype=np.int64) % 251).astype(np.uint8).reshape(M, K // 2)
    scales = (np.arange(M * K // 16, dtype=np.int64) % 241).astype(np.uint8).reshape(M, K // 16)
    t = tile_ref(codes, scales).reshape(2, 2, 2304)
    # block (t=1, s=1), lane l = c + 16g with c=3, g=2, half h=1, j=2
    c_, g_, h_, j_ = 3, 2, 1, 2
    row, b0 = 16 + c_, 128 + 64 * h_ + 16 * j_ + 4 * g_
    off = 1024 * h_ + 16 * (c_ + 16 * g_) + 4 * j_
    assert np.array_equal(t[1, 1, off:off + 4], codes[row, b0:b0 + 4])
    # scale of row 16 + 3 for block 16 + 8 + 2*1 + 1 lands at 2048 + 8*(16 + 3) + 4 + 1
    assert t[1, 1, 2048 + 8 * (16 + 3) + 4 + 1] == scales[19, 16 + 8 + 2 + 1]
    # padding rows (M = 20 < 32) are zero
    assert not t[1, :, :2048].reshape(2, 2, 64, 16)[:, :, [l for l in range(64) if (l & 15) >= 4], :].any()


@pytest.mark.parametrize("M,K", [(1, 16), (16, 128), (17, 48), (40, 528), (33, 1040)])
def test_fp8_tile_ref_round_trip(M, K):
    d = inputs.fp8row_inputs(M, K, 1, seed=M * 5 + K)
    t = fp8_tile_ref(d.w)
    assert t.size == -(-M // 16) * -(-K // 128) * 2048
    assert np.array_equal(fp8_untile_ref(t, M, K), d.w)


def test_fp8_tile_ref_places_bytes_as_documented():
    M, K = 20, 256
    w = (np.arange(M * K, dtype=np.int64) % 253).astype(np.uint8).reshape(M, K)
    t = fp8_tile_ref(w).reshape(2, 2, 2048)
    # block (t=1, s=1), lane l = c + 16g with c=3, g=2, half h=1
    c_, g_, h_ = 3, 2, 1
    row, k0 = 16 + c_, 128 + 64 * h_ + 16 * g_
    off = 1024 * h_ + 16 * (c_ + 16 * g_)
    assert np.array_equal(t[1, 1, off:off + 16], w[row, k0:k0 + 16])
    # every byte of the plain matrix appears exactly once; the rest is padding
    assert np.array_equal(np.sort(t[t != 0]), np.sort(w[w != 0].reshape(-1)))
