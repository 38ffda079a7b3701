"""Pins of the oracle's OCP E5M2 codec and of the E5M2-activation quantizer and linear.

Page "FP8量化在生成式推荐系统OneRec-V2中的优化实践", §2.2, quantizes activations to E5M2
while weights stay E4M3.  The codec is pinned against the OCP OFP8 definition (spec points,
counts), PyTorch's independent float8_e5m2 conversion (all FP16 values, random FP32) and a
brute-force nearest-value search; the quantizer against closed forms; the linear against
exact rational arithmetic.
"""

from fractions import Fraction

import numpy as np
import torch

from oracle import e4m3, e5m2, linear, quant

ALL_FP16 = np.arange(65536, dtype=np.uint16).view(np.float16)
FINITE_FP16 = ALL_FP16[np.isfinite(ALL_FP16)]
POS_FP16 = np.unique(FINITE_FP16[FINITE_FP16 > 0])
E5M2_FINITE = np.array([c for c in range(256) if (c & 0x7C) != 0x7C], np.uint8)
E4M3_FINITE = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)


def _torch_decode_all():
    return torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e5m2).to(torch.float64).numpy()


def test_spec_points():
    # OCP OFP8 E5M2: bias 15, subnormal step 2^-16, IEEE-style infinities and NaNs
    tab = e5m2.table()
    assert tab[0x00] == 0.0 and not np.signbit(tab[0x00])
    assert tab[0x80] == 0.0 and np.signbit(tab[0x80])
    assert tab[0x01] == 2.0 ** -16 and tab[0x03] == 3 * 2.0 ** -16
    assert tab[0x04] == 2.0 ** -14                       # smallest normal
    assert tab[0x3C] == 1.0 and tab[0xBC] == -1.0
    assert tab[0x3D] == 1.25 and tab[0x3F] == 1.75
    assert tab[0x7B] == 57344.0 and tab[0xFB] == -57344.0
    assert tab[0x7C] == np.inf and tab[0xFC] == -np.inf
    assert all(np.isnan(tab[c]) for c in (0x7D, 0x7E, 0x7F, 0xFD, 0xFE, 0xFF))


def test_decode_matches_torch_all_codes():
    ours, ref = e5m2.table(), _torch_decode_all()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin], ref[fin])
    assert np.array_equal(np.signbit(ours[fin]), np.signbit(ref[fin]))


def test_code_counts():
    tab = e5m2.table()
    fin = tab[np.isfinite(tab)]
    assert fin.size == 248 and np.sum(fin > 0) == 123
    assert np.max(fin) == e5m2.MAX_FINITE


def test_roundtrip_all_finite_codes():
    vals = e5m2.decode(E5M2_FINITE)
    assert np.array_equal(e5m2.encode(vals), E5M2_FINITE)


def test_saturation_nan_and_signed_zero():
    v = np.array([57344.0, 57345.0, 61440.0, 1e30, np.inf, -57344.0, -np.inf, np.nan, -0.0, -(2.0 ** -18)])
    q = e5m2.encode(v)
    assert q[:5].tolist() == [0x7B] * 5
    assert q[5:7].tolist() == [0xFB] * 2
    assert (q[7] & 0x7C) == 0x7C and (q[7] & 0x03) != 0
    assert q[8:].tolist() == [0x80, 0x80]                 # a quarter step rounds to -0


def test_all_fp16_values_match_torch_within_range():
    v = FINITE_FP16.astype(np.float64)
    ok = np.abs(v) <= 57344.0
    ref = torch.from_numpy(v[ok].astype(np.float32)).to(torch.float8_e5m2).view(torch.uint8).numpy()
    assert np.array_equal(e5m2.encode(v[ok]), ref)
    big = e5m2.encode(v[~ok])
    assert np.all((big & 0x7F) == 0x7B)


def test_random_fp32_match_torch():
    rng = np.random.default_rng(5)
    v = (rng.standard_normal(300000) * np.exp2(rng.uniform(-20, 16, 300000))).astype(np.float32).astype(np.float64)
    ok = np.abs(v) <= 57344.0
    ref = torch.from_numpy(v[ok].astype(np.float32)).to(torch.float8_e5m2).view(torch.uint8).numpy()
    assert np.array_equal(e5m2.encode(v[ok]), ref)


def test_brute_force_nearest_with_ties_to_even():
    pos = np.sort(e5m2.decode(E5M2_FINITE[(E5M2_FINITE < 0x80)]))
    mids = (pos[:-1] + pos[1:]) / 2
    q = e5m2.encode(mids)
    lo, hi = e5m2.encode(pos[:-1]), e5m2.encode(pos[1:])
    assert np.array_equal(q, np.where(lo % 2 == 0, lo, hi))  # each midpoint takes the even byte
    eps = np.nextafter(mids, np.inf) - mids
    assert np.array_equal(e5m2.encode(mids + eps), hi)
    assert np.array_equal(e5m2.encode(mids - eps), lo)


def test_e5m2_amax_maps_to_57344_for_every_fp16_amax():
    rows = np.stack([POS_FP16, -POS_FP16, POS_FP16 * np.float16(0.25)], axis=1)
    q, s = quant.quantize_rows(rows, "e5m2")
    assert np.all(q[:, 0] == 0x7B) and np.all(q[:, 1] == 0xFB)


def test_e5m2_scale_is_the_e4m3_scale_over_128():
    # 57344 = 448 * 128, so fl32(amax / 57344) = fl32(amax / 448) / 128 exactly, for every
    # FP16 amax, and the FP32 quotients scale by 128 exactly as well.
    s4 = quant.row_scale(POS_FP16.astype(np.float64))
    s5 = quant.row_scale(POS_FP16.astype(np.float64), e5m2.MAX_FINITE)
    assert np.array_equal(s5.astype(np.float64) * 128, s4.astype(np.float64))
    ref = (torch.from_numpy(POS_FP16.astype(np.float32)) / torch.tensor(57344.0, dtype=torch.float32)).numpy()
    assert np.array_equal(s5.view(np.uint32), ref.view(np.uint32))


def test_e5m2_exhaustive_fp16_at_unit_scale():
    v = FINITE_FP16[np.abs(FINITE_FP16.astype(np.float64)) <= 57344.0]
    rows = np.stack([np.full(v.shape, 57344.0, np.float16), v], axis=1)
    q, s = quant.quantize_rows(rows, "e5m2")
    assert np.all(s == np.float32(1.0))
    ref = torch.from_numpy(v.astype(np.float32)).to(torch.float8_e5m2).view(torch.uint8).numpy()
    assert np.array_equal(q[:, 1], ref)


def test_e5m2_linear_matches_exact_rational_brute_force():
    rng = np.random.default_rng(9)
    m, n, k = 3, 5, 40
    xq = rng.choice(E5M2_FINITE, size=(m, k)).astype(np.uint8)
    wq = rng.choice(E4M3_FINITE, size=(n, k)).astype(np.uint8)
    xq[0, 0], wq[0, 0] = 0x7B, 0x7E                         # 57344 * 448
    xq[1, 1], wq[1, 1] = 0x01, 0x81                         # the smallest subnormal product
    acc = linear.gemm_exact(xq, wq, "e5m2")
    a5, a4 = e5m2.decode(xq), e4m3.decode(wq)
    for i in range(m):
        for j in range(n):
            exact = sum(Fraction(float(a5[i, t])) * Fraction(float(a4[j, t])) for t in range(k))
            assert Fraction(acc[i, j]) == exact


def test_e5m2_exact_at_largest_k():
    # K = 8192 products of +/-57344 * 448: sums beyond 2^53 units, exact through int64
    xq = np.full((2, 8192), 0x7B, np.uint8)
    xq[1, ::2] = 0xFB
    wq = np.full((1, 8192), 0x7E, np.uint8)
    wq[0, 1] = 0x01                                          # the smallest E4M3 subnormal
    acc = linear.gemm_exact(xq, wq, "e5m2")
    exact0 = Fraction(8191 * 57344 * 448) + Fraction(57344) * Fraction(1, 512)
    assert Fraction(acc[0, 0]) == exact0
    exact1 = -Fraction(4096 * 57344 * 448) + Fraction(4095 * 57344 * 448) + Fraction(57344, 512)
    assert Fraction(acc[1, 0]) == exact1
