"""Pins of the oracle's per-tensor and 128 x 128 block weight scales (oracle.wscale).

Page "FP8量化在生成式推荐系统OneRec-V2中的优化实践", §2.1 / §2.2: the dense FFN weights
carry one scale per tensor, the MoE expert weights one scale per 128 x 128 block.  The
pins reduce each variant to the pinned row quantizer and linear in the cases where they
must agree, check closed forms, and brute-force the block linear over exact rationals.
"""

from fractions import Fraction

import numpy as np
import pytest

from oracle import e4m3, linear, moe, quant, wscale

FINITE_CODES = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)


def _frac_decode(c):
    c = int(c)
    s = -1 if c & 0x80 else 1
    e = (c >> 3) & 15
    m = c & 7
    if e == 0:
        return s * Fraction(m, 512)
    return s * Fraction(8 + m) * (Fraction(2) ** (e - 10))


def _weights(rng, n, k, std=0.02):
    return (rng.standard_normal((n, k)) * std).astype(np.float16)


def test_tensor_scale_is_the_row_scale_when_every_row_holds_the_maximum():
    rng = np.random.default_rng(11)
    w = _weights(rng, 96, 160)
    peak = np.float16(0.125)
    for r in range(w.shape[0]):
        w[r, rng.integers(0, w.shape[1])] = peak if r % 2 else -peak
    q_t, s_t = wscale.quantize_tensor(w)
    q_r, s_r = quant.quantize_rows(w)
    assert s_t.shape == (1,) and s_t.dtype == np.float32
    assert np.all(s_r == s_t[0])
    assert np.array_equal(q_t, q_r)


def test_block_scales_are_the_row_scales_of_rows_that_hold_the_block_maximum():
    rng = np.random.default_rng(12)
    n, k = 256, 384
    w = _weights(rng, n, k)
    peaks = rng.uniform(0.2, 0.5, size=(n // 128, k // 128)).astype(np.float16)  # > 10 sigma
    for i in range(n // 128):
        for j in range(k // 128):
            for r in range(128 * i, 128 * i + 128):
                w[r, 128 * j + rng.integers(0, 128)] = peaks[i, j] * (1 if r % 3 else -1)
    q_b, s_b = wscale.quantize_blocks(w)
    assert s_b.shape == (2, 3) and s_b.dtype == np.float32
    for i in range(2):
        for j in range(3):
            rows, cols = slice(128 * i, 128 * i + 128), slice(128 * j, 128 * j + 128)
            q_r, s_r = quant.quantize_rows(w[rows, cols])
            assert np.all(s_r == s_b[i, j])
            assert np.array_equal(q_b[rows, cols], q_r)


def test_power_of_two_blocks_are_exact_and_keep_their_own_scale():
    # Block (i, j) holds E4M3 values times 2^p[i, j] including +-448 * 2^p: its scale is
    # exactly 2^p[i, j] and the codes come back unchanged.  Distinct exponents per block
    # catch a transposed or shifted block index.
    rng = np.random.default_rng(13)
    p = np.array([[-9, -6, -12], [-7, -10, -8]])
    codes = rng.choice(FINITE_CODES, size=(256, 384)).astype(np.uint8)
    codes[::128, ::128] = 0x7E
    vals = e4m3.decode(codes) * np.repeat(np.repeat(2.0 ** p, 128, 0), 128, 1)
    w = vals.astype(np.float16)
    assert np.array_equal(w.astype(np.float64), vals)       # representable in FP16
    q_b, s_b = wscale.quantize_blocks(w)
    assert np.array_equal(s_b.astype(np.float64), 2.0 ** p)
    # -0 encodes as 0x80 from a negative zero value only; compare through the values
    assert np.array_equal(e4m3.decode(q_b), e4m3.decode(codes))


def test_block_quantization_error_bound():
    rng = np.random.default_rng(14)
    w = _weights(rng, 128, 256, std=0.05)
    w[5, 7] = np.float16(3e-6)                                # deep in the subnormal range
    q, s = wscale.quantize_blocks(w)
    S = np.repeat(np.repeat(s.astype(np.float64), 128, 0), 128, 1)
    x = w.astype(np.float64)
    err = np.abs(x - e4m3.decode(q) * S)
    normal = np.abs(x / S) >= 2.0 ** -6
    assert np.all(err[normal] <= (2.0 ** -4 + 2.0 ** -23) * np.abs(x[normal]))
    assert np.all(err[~normal] <= 2.0 ** -10 * S[~normal] + 2.0 ** -23 * np.abs(x[~normal]))


def test_block_shapes_must_be_multiples_of_128():
    with pytest.raises(ValueError):
        wscale.quantize_blocks(np.zeros((128, 192), np.float16))
    with pytest.raises(ValueError):
        wscale.quantize_blocks(np.zeros((64, 128), np.float16))


def test_zero_block_takes_the_floor_scale():
    w = np.zeros((128, 256), np.float16)
    w[:, 128:] = np.float16(0.5)
    q, s = wscale.quantize_blocks(w)
    assert s[0, 0] == np.float32(2.0 ** -24 / 448.0)
    assert np.all(q[:, :128] == 0)
    assert s[0, 1] == np.float32(0.5 / 448.0)


def test_block_linear_matches_exact_rational_brute_force():
    rng = np.random.default_rng(15)
    m, n, k = 2, 256, 256
    xq = rng.choice(FINITE_CODES, size=(m, k)).astype(np.uint8)
    wq = rng.choice(FINITE_CODES, size=(n, k)).astype(np.uint8)
    s_x = np.array([0.0123, 3.5e-3], np.float32)
    S = np.array([[1.5e-4, 7.0e-3], [2.0 ** -12, 9.1e-4]], np.float32)
    y = wscale.linear(xq, s_x, wq, S, wscale.BLOCK128)
    for i in range(m):
        for c in range(0, n, 37):
            exact = Fraction(0)
            for j in range(2):
                part = sum(_frac_decode(xq[i, t]) * _frac_decode(wq[c, t]) for t in range(128 * j, 128 * j + 128))
                exact += Fraction(float(S[c // 128, j])) * part
            exact *= Fraction(float(s_x[i]))
            assert y[i, c] == np.float16(float(exact))


def test_block_linear_with_scales_constant_along_k_is_the_per_channel_linear():
    rng = np.random.default_rng(16)
    xq = rng.choice(FINITE_CODES, size=(5, 384)).astype(np.uint8)
    wq = rng.choice(FINITE_CODES, size=(256, 384)).astype(np.uint8)
    s_x = rng.uniform(1e-3, 1e-2, size=5).astype(np.float32)
    per_block_row = np.array([2.0 ** -9, 2.0 ** -11], np.float32)   # powers of two: exact products
    S = np.repeat(per_block_row[:, None], 3, axis=1)
    s_w = np.repeat(per_block_row, 128)
    y_b = wscale.linear(xq, s_x, wq, S, wscale.BLOCK128)
    y_c = linear.linear(xq, s_x, wq, s_w)
    assert np.array_equal(y_b, y_c)


def test_tensor_linear_is_the_per_channel_linear_with_one_repeated_scale():
    rng = np.random.default_rng(17)
    xq = rng.choice(FINITE_CODES, size=(4, 64)).astype(np.uint8)
    wq = rng.choice(FINITE_CODES, size=(48, 64)).astype(np.uint8)
    s_x = rng.uniform(1e-3, 1e-2, size=4).astype(np.float32)
    s = np.array([3.3e-4], np.float32)
    assert np.array_equal(wscale.linear(xq, s_x, wq, s, wscale.TENSOR),
                          linear.linear(xq, s_x, wq, np.full(48, s[0], np.float32)))


def test_block_check_accepts_the_reference_and_rejects_a_wrong_block_scale():
    rng = np.random.default_rng(18)
    w = _weights(rng, 256, 256)
    w[:128, :128] *= np.float16(4.0)                          # blocks with clearly different scales
    wq, S = wscale.quantize_blocks(w)
    xq, s_x = quant.quantize_rows(_weights(rng, 6, 256, std=1.0))
    ok, ratio, y_ref = wscale.check(wscale.linear(xq, s_x, wq, S, wscale.BLOCK128), xq, s_x, wq, S, wscale.BLOCK128)
    assert ok and ratio == 0.0
    swapped = S[:, ::-1].copy()                               # K blocks in the wrong order
    ok, ratio, _ = wscale.check(wscale.linear(xq, s_x, wq, swapped, wscale.BLOCK128), xq, s_x, wq, S,
                                wscale.BLOCK128)
    assert not ok


def test_moe_on_one_expert_is_the_dense_block_linear():
    rng = np.random.default_rng(19)
    t, k, n, e = 12, 256, 128, 3
    x = rng.standard_normal((t, k)).astype(np.float16)
    ids = np.zeros((t, 1), np.int32) + 2
    wq = np.zeros((e, n, k), np.uint8)
    ws = np.zeros((e, n // 128, k // 128), np.float32)
    for i in range(e):
        wq[i], ws[i] = wscale.quantize_blocks(_weights(rng, n, k))
    r = moe.grouped_linear(x, moe.IN_TOKENS, moe.ACT_NONE, ids, wq, ws, gran=wscale.BLOCK128)
    xq, sx = quant.quantize_rows(x)
    assert np.array_equal(r["y"], wscale.linear(xq, sx, wq[2], ws[2], wscale.BLOCK128))
