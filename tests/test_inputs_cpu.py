"""The seeded input generators (no GPU): the hashed-row generators give the
same bytes for a row however the rows are chunked, distinct rows, block
scales only from their table, FP8 codes without NaN and row scales in their
stated range."""
import numpy as np

from fp8_weight_streaming_amd import inputs


def test_hashed_rows_do_not_depend_on_chunking():
    K = 544
    c_all, s_all = inputs.hashed_nvfp4_rows(np.arange(0, 300), K, seed=11)
    c_sub, s_sub = inputs.hashed_nvfp4_rows(np.array([7, 299, 150]), K, seed=11)
    assert np.array_equal(c_sub, c_all[[7, 299, 150]]) and np.array_equal(s_sub, s_all[[7, 299, 150]])
    w_all, r_all = inputs.hashed_fp8_rows(np.arange(0, 300), 272, seed=12)
    w_sub, r_sub = inputs.hashed_fp8_rows(np.array([0, 123]), 272, seed=12)
    assert np.array_equal(w_sub, w_all[[0, 123]]) and np.array_equal(r_sub, r_all[[0, 123]])
    # another seed gives other bytes
    assert not np.array_equal(inputs.hashed_nvfp4_rows(np.arange(0, 4), K, seed=13)[0], c_all[:4])


def test_hashed_rows_are_distinct_and_in_range():
    c, s = inputs.hashed_nvfp4_rows(np.arange(0, 4096), 1024, seed=5)
    assert len({r.tobytes() for r in c}) == 4096
    table = {((e + 7) << 3) | m for e in range(-4, 4) for m in (0, 4)}
    assert set(np.unique(s).tolist()) <= table and len(np.unique(s)) == 16
    # codes spread over every byte value, nibbles near uniform
    hist = np.bincount((c & 15).ravel(), minlength=16) / c.size
    assert np.unique(c).size == 256 and np.abs(hist - 1 / 16).max() < 0.005
    w, r = inputs.hashed_fp8_rows(np.arange(0, 4096), 512, seed=6)
    assert not (w & 0x08).any()  # the lowest exponent bit clear: no S.1111.111 (NaN) code
    assert ((r >= 2.0 ** -10) & (r <= 2.0 ** -10 * 1.875)).all() and len(np.unique(r)) == 8
