"""Pins of the oracle's E4M3 codec against the OCP definition and an independent library.

* the format's printed points (``tests/golden/e4m3_ocp_points.txt``, from the OCP OFP8
  specification's E4M3 column; the +/-448 range also appears on page
  "FP8量化在生成式推荐系统OneRec-V2中的优化实践", §1.2);
* PyTorch's own CPU float8_e4m3fn conversion, written independently of this code;
* a brute-force nearest-value search with ties to even over the 254 finite values.
"""

import os

import numpy as np
import pytest
import torch

from oracle import e4m3

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_ocp_points.txt")


def _golden_points():
    pts = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            code, value = line.split()[:2]
            pts.append((int(code, 16), float(value)))
    return pts


def _torch_decode_all():
    return torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_spec_points():
    tab = e4m3.table()
    for code, value in _golden_points():
        if np.isnan(value):
            assert np.isnan(tab[code]), hex(code)
        else:
            assert tab[code] == value, hex(code)
            assert np.signbit(tab[code]) == np.signbit(value), hex(code)


def test_decode_matches_torch_all_codes():
    ours = e4m3.table()
    ref = _torch_decode_all()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin], ref[fin])
    assert np.array_equal(np.signbit(ours[fin]), np.signbit(ref[fin]))


def test_code_counts_and_extremes():
    tab = e4m3.table()
    fin = tab[~np.isnan(tab)]
    assert fin.size == 254
    assert np.sum(fin > 0) == 126
    assert np.max(fin) == 448.0 and np.argmax(np.nan_to_num(tab, nan=-1)) == 0x7E
    assert np.min(fin) == -448.0
    assert sorted(np.flatnonzero(np.isnan(tab)).tolist()) == [0x7F, 0xFF]
    pos = np.sort(fin[fin > 0])
    assert pos[0] == 2.0 ** -9 and pos[7] == 2.0 ** -6


def test_roundtrip_all_finite_codes():
    codes = np.arange(256, dtype=np.uint8)
    vals = e4m3.decode(codes)
    fin = ~np.isnan(vals)
    assert np.array_equal(e4m3.encode(vals[fin]), codes[fin])


def test_nan_and_saturation():
    v = np.array([np.nan, -np.nan, 448.0, 448.5, 464.0, 1e30, np.inf, -448.0, -1e9, -np.inf])
    q = e4m3.encode(v)
    assert q[0] & 0x7F == 0x7F and q[1] & 0x7F == 0x7F
    assert q[2:7].tolist() == [0x7E] * 5
    assert q[7:].tolist() == [0xFE] * 3


def test_signed_zero_and_negative_underflow():
    v = np.array([0.0, -0.0, 2.0 ** -11, -(2.0 ** -11), -(2.0 ** -10)])
    # 2^-11 is a quarter unit of 2^-9: rounds to 0, keeping the sign.
    # 2^-10 is half a unit: the tie goes to the even neighbour, 0.
    assert e4m3.encode(v).tolist() == [0x00, 0x80, 0x00, 0x80, 0x80]


def test_all_fp16_values_match_torch_below_448():
    h = np.arange(65536, dtype=np.uint16).view(np.float16)
    v = h.astype(np.float64)
    ok = np.isfinite(v) & (np.abs(v) < 448.0)
    ours = e4m3.encode(v[ok])
    ref = torch.from_numpy(v[ok].astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)
    big = np.isfinite(v) & (np.abs(v) >= 448.0)
    qb = e4m3.encode(v[big])
    assert np.all((qb == 0x7E) | (qb == 0xFE))
    assert np.array_equal(qb >> 7, np.signbit(v[big]).astype(np.uint8))


def test_random_fp32_match_torch():
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 2 ** 32, size=400000, dtype=np.uint64).astype(np.uint32)
    v32 = bits.view(np.float32)
    with np.errstate(invalid="ignore"):
        v = v32.astype(np.float64)
    ok = np.isfinite(v) & (np.abs(v) < 448.0)
    # also a dense sample over the format's own range
    dense = (rng.standard_normal(400000) * np.exp2(rng.uniform(-12, 8.8, 400000))).astype(np.float32)
    dense = dense[np.abs(dense) < 448.0].astype(np.float64)
    for arr in (v[ok], dense):
        ref = torch.from_numpy(arr.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(e4m3.encode(arr), ref)


def _brute_nearest_even(x):
    """Nearest E4M3 magnitude by exhaustive search over bytes 0x00..0x7E, ties to the
    even byte, the input's sign kept; saturation at 448."""
    sign = 0x80 if np.signbit(x) else 0x00
    if abs(x) >= 448.0:
        return 0x7E | sign
    codes = np.arange(0x7F)
    mags = e4m3.decode(codes.astype(np.uint8))
    d = np.abs(mags - abs(x))
    cand = codes[d == d.min()]
    even = [c for c in cand if c % 2 == 0]
    return int(even[0] if even else cand[0]) | sign


def test_brute_force_nearest_with_midpoints():
    tab = e4m3.table()
    pos = np.sort(tab[(~np.isnan(tab)) & (tab > 0)])
    mids = (pos[:-1] + pos[1:]) / 2.0
    rng = np.random.default_rng(11)
    xs = list(mids) + list(-mids) + list(rng.uniform(-460, 460, 3000)) + \
        list(rng.standard_normal(2000) * 2.0 ** -7) + [2.0 ** -10, 3 * 2.0 ** -10, 447.99]
    xs = np.array(xs, dtype=np.float64)
    got = e4m3.encode(xs)
    for x, g in zip(xs, got):
        assert int(g) == _brute_nearest_even(float(x)), (x, hex(int(g)))


@pytest.mark.parametrize("code", [0x01, 0x07, 0x08, 0x38, 0x39, 0x77, 0x7D])
def test_ties_go_to_even_byte(code):
    lo, hi = e4m3.decode(np.array([code, code + 1], np.uint8))
    q = int(e4m3.encode(np.array([(lo + hi) / 2.0]))[0])
    assert q in (code, code + 1) and q % 2 == 0
