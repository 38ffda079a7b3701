"""Slab layout of quantized weights.  Test infrastructure.

The pages fix no byte layout for the quantized weights beyond one E4M3 byte per weight; the
slab layout is this library's own, chosen for how the GEMM streams weights from HBM.  It is a
permutation of the bytes of each [N][K] matrix: the columns are cut into slabs of 64
(columns 64s .. 64s + 63); slab s of the matrix - an N x 64 slice - is stored row by row
(N runs of 64 bytes), slab 0 first, then slab 1, and so on.  A stack of B matrices stores
them one after another.

Defined by those slices, in that order, and nothing else; no arithmetic on values.
"""

import numpy as np

SLAB = 64


def pack_slabs(w_q):
    """uint8 [N, K] or [B, N, K] (row layout) -> flat uint8 array of the slab layout."""
    w = np.asarray(w_q, dtype=np.uint8)
    if w.ndim == 2:
        w = w[None]
    if w.ndim != 3:
        raise ValueError("w_q must be [N, K] or [B, N, K]")
    b, n, k = w.shape
    if k % SLAB:
        raise ValueError("K must be a multiple of 64")
    pieces = []
    for m in range(b):
        for s in range(k // SLAB):
            pieces.append(w[m, :, s * SLAB:(s + 1) * SLAB].reshape(-1))  # the N x 64 slice, row by row
    return np.concatenate(pieces) if pieces else np.zeros(0, np.uint8)


def unpack_slabs(flat, b, n, k):
    """Inverse of ``pack_slabs``: the [B, N, K] row layout."""
    flat = np.asarray(flat, dtype=np.uint8).reshape(-1)
    if flat.size != b * n * k:
        raise ValueError("size mismatch")
    w = np.empty((b, n, k), np.uint8)
    at = 0
    for m in range(b):
        for s in range(k // SLAB):
            w[m, :, s * SLAB:(s + 1) * SLAB] = flat[at:at + n * SLAB].reshape(n, SLAB)
            at += n * SLAB
    return w
