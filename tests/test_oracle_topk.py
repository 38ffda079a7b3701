"""Pins of ``oracle.topk`` (CPU only): the ranking is checked against definitions that do not
use the oracle's key encoding - Python's own sort of (value, sign, index) tuples, numpy's
stable argsort, PyTorch's topk on distinct values, planted winners - and the two-stage
reading (top-k of segment-wise top-k candidates) is checked to give the same result."""

import numpy as np
import pytest
import torch
from hypothesis import given, settings
from hypothesis import strategies as st

from oracle import topk


def _brute(row16, k):
    """Rank by (value descending, +0 before -0, index ascending) with Python's sort."""
    vals = [float(v) for v in row16]
    signs = [int(np.signbit(v)) for v in row16]  # -0 has the sign bit: it ranks below +0
    order = sorted(range(len(vals)), key=lambda i: (-vals[i], signs[i] if vals[i] == 0 else 0, i))
    return np.array(order[:k])


def test_key_order_is_the_value_order_on_every_fp16():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = bits.view(np.float16)
    ok = ~np.isnan(vals)
    bits, vals = bits[ok], vals[ok]
    keys = topk.order_key(bits)
    assert np.unique(keys).size == bits.size                      # one key per pattern
    by_key = np.argsort(keys, kind="stable")
    v = vals[by_key].astype(np.float64)
    assert np.all(np.diff(v) >= 0)                                # keys sort by value
    zero = np.where(v == 0)[0]
    assert zero.size == 2 and np.signbit(vals[by_key][zero[0]]) and not np.signbit(vals[by_key][zero[1]])
    assert np.array_equal(topk.from_key(keys), bits)


@pytest.mark.parametrize("seed", range(6))
def test_brute_force_with_ties_and_signed_zeros(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 70))
    pool = np.array([0.0, -0.0, 1.0, -1.0, 0.5, 2.0, -3.0, 65504.0, -65504.0, 6e-8, -6e-8], np.float16)
    rows = pool[rng.integers(0, pool.size, size=(3, n))]
    for k in sorted({1, max(1, n // 2), n}):
        idx, vals = topk.topk(rows, k)
        for r in range(rows.shape[0]):
            ref = _brute(rows[r], k)
            assert np.array_equal(idx[r], ref)
            assert np.array_equal(vals[r].view(np.uint16), rows[r][ref].view(np.uint16))


@settings(max_examples=60, deadline=None)
@given(st.integers(1, 200), st.integers(0, 2 ** 31 - 1))
def test_full_sort_is_the_stable_descending_sort(n, seed):
    rng = np.random.default_rng(seed)
    row = (rng.standard_normal(n) * 4).astype(np.float16)
    row[row == 0] = np.float16(0.0)  # one zero sign: value ties are then index ties only
    idx, _ = topk.topk(row[None], n)
    assert np.array_equal(idx[0], np.argsort(-row.astype(np.float64), kind="stable"))


def test_matches_torch_topk_on_distinct_values():
    rng = np.random.default_rng(5)
    row = rng.permutation(np.arange(-2048, 2048)).astype(np.float16)  # distinct, exact in FP16
    for k in (1, 16, 512, 4096):
        idx, vals = topk.topk(row[None], k)
        tv, ti = torch.topk(torch.from_numpy(row.astype(np.float32)), k)
        assert np.array_equal(idx[0], ti.numpy()) and np.array_equal(vals[0].astype(np.float32), tv.numpy())


def test_planted_winners_and_permutation():
    rng = np.random.default_rng(9)
    n, k = 5000, 37
    row = (rng.random(n) * 10).astype(np.float16)
    where = rng.choice(n, size=k, replace=False)
    row[where] = (100 + np.arange(k)).astype(np.float16)  # distinct, all above the rest
    idx, vals = topk.topk(row[None], k)
    assert np.array_equal(idx[0], where[::-1])             # 100 + k - 1 first
    perm = rng.permutation(n)
    idx_p, _ = topk.topk(row[perm][None], k)
    assert np.array_equal(perm[idx_p[0]], idx[0])          # permuting candidates permutes the picks


def test_all_equal_row_takes_the_lowest_indices():
    row = np.full((2, 300), 1.25, np.float16)
    idx, vals = topk.topk(row, 20)
    assert np.array_equal(idx, np.tile(np.arange(20), (2, 1))) and np.all(vals == 1.25)


@pytest.mark.parametrize("seg", [1, 7, 64, 1000])
def test_top_k_of_segment_candidates_equals_top_k(seg):
    """Staged selection: every member of the row's top k is in its own segment's top k (at
    most k - 1 candidates of the whole row rank before it), so the top k of the union of the
    segments' top k is the row's top k."""
    rng = np.random.default_rng(seg)
    n, k = 3000, 50
    row = rng.integers(-20, 20, size=n).astype(np.float16)  # many ties
    want_idx, want_vals = topk.topk(row[None], k)
    cand_idx = []
    for lo in range(0, n, seg):
        part = row[lo:lo + seg]
        ci, _ = topk.topk(part[None], min(k, part.size))
        cand_idx.append(ci[0] + lo)
    cand = np.concatenate(cand_idx)          # ascending segment order keeps index order per value
    ci, cv = topk.topk(row[cand][None], k)
    assert np.array_equal(cand[ci[0]], want_idx[0]) and np.array_equal(cv, want_vals)


def test_rejects_bad_k_and_nan():
    with pytest.raises(ValueError):
        topk.topk(np.zeros((1, 4), np.float16), 5)
    with pytest.raises(ValueError):
        topk.topk(np.zeros((1, 4), np.float16), 0)
    with pytest.raises(ValueError):
        topk.topk(np.array([[np.nan, 1]], np.float16), 1)
