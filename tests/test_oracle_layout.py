"""Pins of ``oracle.layout`` (CPU only): the slab layout is pinned against its stated
properties - a byte permutation whose inverse restores the matrix, where each run of 64 N
bytes holds one N x 64 column slice, and where chosen bytes land at positions worked out by
hand - rather than against a retyped formula."""

import numpy as np
import pytest

from oracle import layout


def test_worked_example_positions():
    # N = 3, K = 128: two slabs of 3 x 64 = 192 bytes.  Byte (n=2, k=65) is in slab 1 (after
    # 192 bytes), row 2 of it (2 * 64 more), column 1: position 192 + 128 + 1 = 321.
    w = np.zeros((3, 128), np.uint8)
    w[2, 65] = 7
    w[0, 0] = 1        # first byte
    w[2, 63] = 2       # last byte of slab 0: 191
    w[0, 64] = 3       # first byte of slab 1: 192
    w[1, 0] = 4        # row 1 of slab 0 follows row 0: 64
    flat = layout.pack_slabs(w)
    assert flat[0] == 1 and flat[191] == 2 and flat[192] == 3 and flat[64] == 4 and flat[321] == 7
    assert np.count_nonzero(flat) == 5
    # a stack: matrix 1 starts after the N * K bytes of matrix 0
    s = np.zeros((2, 3, 128), np.uint8)
    s[1, 0, 0] = 9
    assert layout.pack_slabs(s)[3 * 128] == 9


@pytest.mark.parametrize("shape", [(1, 1, 64), (2, 5, 192), (3, 384, 128), (2, 130, 256)])
def test_permutation_and_inverse(shape):
    b, n, k = shape
    rng = np.random.default_rng(b * n + k)
    w = rng.integers(0, 256, size=shape, dtype=np.uint8)
    flat = layout.pack_slabs(w)
    assert flat.size == w.size
    assert np.array_equal(layout.unpack_slabs(flat, b, n, k), w)          # inverse restores
    # position tags: packing the position index shows a bijection of positions
    pos = np.arange(w.size)
    tags = [(pos >> (8 * j)) & 0xFF for j in range(3)]
    packed = [layout.pack_slabs(t.astype(np.uint8).reshape(shape)).astype(np.int64) for t in tags]
    src = packed[0] | (packed[1] << 8) | (packed[2] << 16)
    assert np.array_equal(np.sort(src), pos)


def test_slabs_are_contiguous_column_slices():
    b, n, k = 2, 200, 256
    w = np.random.default_rng(3).integers(0, 256, size=(b, n, k), dtype=np.uint8)
    flat = layout.pack_slabs(w).reshape(b, k // 64, n, 64)
    for m in range(b):
        for s in range(k // 64):
            assert np.array_equal(flat[m, s], w[m, :, 64 * s:64 * s + 64])


def test_one_slab_is_the_row_layout():
    # K = 64: a single slab, stored row by row - the row layout itself
    w = np.random.default_rng(1).integers(0, 256, size=(300, 64), dtype=np.uint8)
    assert np.array_equal(layout.pack_slabs(w), w.reshape(-1))
    # a single row: its slabs in order - again the row itself
    w = np.random.default_rng(2).integers(0, 256, size=(1, 320), dtype=np.uint8)
    assert np.array_equal(layout.pack_slabs(w), w.reshape(-1))


def test_rejects_unaligned():
    with pytest.raises(ValueError):
        layout.pack_slabs(np.zeros((128, 48), np.uint8))
