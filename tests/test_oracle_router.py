"""Pins of the oracle's MoE router (FP16 gate logits, top-k selection, softmax weights).

Page "FP8量化在生成式推荐系统OneRec-V2中的优化实践", §2.1: the routing gate stays FP16; its
top-k result feeds the MoE grouped GEMM.  Pinned by exact rational logits, library argmax /
lexsort on the selection, closed-form softmax weights and an FP32 accumulation check of the
error bound.
"""

import math
from fractions import Fraction

import numpy as np

from oracle import router


def test_logits_match_rational_brute_force():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((3, 48)).astype(np.float16)
    w = (rng.standard_normal((5, 48)) * 0.05).astype(np.float16)
    w[0, 0] = np.float16(6e-8)                                # an FP16 subnormal
    lg = router.logits(x, w)
    for i in range(3):
        for e in range(5):
            exact = sum(Fraction(float(x[i, k])) * Fraction(float(w[e, k])) for k in range(48))
            assert abs(Fraction(lg[i, e]) - exact) <= abs(exact) * Fraction(48, 2 ** 53) + Fraction(1, 2 ** 1000)


def test_top1_is_numpy_argmax_and_full_order_is_lexsort():
    rng = np.random.default_rng(2)
    lg = rng.standard_normal((200, 32)).round(1)             # rounding makes ties common
    ids1 = router.select(lg, 1)
    assert np.array_equal(ids1[:, 0], np.argmax(lg, axis=1))  # argmax takes the first maximum
    full = router.select(lg, 32)
    idx = np.broadcast_to(np.arange(32), lg.shape)
    ref = np.stack([np.lexsort((idx[r], -lg[r])) for r in range(lg.shape[0])])
    assert np.array_equal(full, ref)


def test_selection_follows_a_permutation_of_experts():
    rng = np.random.default_rng(3)
    lg = rng.standard_normal((50, 16))                        # distinct values, no ties
    perm = rng.permutation(16)
    ids = router.select(lg, 3)
    ids_p = router.select(lg[:, perm], 3)
    assert np.array_equal(perm[ids_p], ids)


def test_weights_closed_forms():
    lg = np.array([[1.0, 1.0, -3.0], [2.0, 0.5, 0.0], [0.0, 0.0, 0.0]])
    ids = router.select(lg, 2)
    w = router.weights(lg, ids)
    assert ids[0].tolist() == [0, 1] and w[0].tolist() == [0.5, 0.5]
    a, b = 2.0, 0.5
    assert w[1, 0] == np.float16(1.0 / (1.0 + math.exp(b - a)))
    assert w[1, 1] == np.float16(1.0 / (1.0 + math.exp(a - b)))
    assert ids[2].tolist() == [0, 1]                          # all equal: lowest indices
    one = router.weights(lg, router.select(lg, 1))
    assert np.all(one == np.float16(1.0))


def test_route_on_a_planted_winner():
    # expert 7's gate row equals the token: its logit is |x|^2, far above the others
    rng = np.random.default_rng(4)
    x = rng.standard_normal((4, 256)).astype(np.float16)
    w = (rng.standard_normal((16, 256)) * 0.01).astype(np.float16)
    w[7] = x[0]
    ids, wts, _ = router.route(x[:1], w, 2)
    assert ids[0, 0] == 7 and wts[0, 0] > np.float16(0.99)


def test_fp32_accumulation_stays_within_the_bound():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((64, 2048)).astype(np.float16)
    w = (rng.standard_normal((32, 2048)) * 0.02).astype(np.float16)
    exact = router.logits(x, w)
    prods = x.astype(np.float32)[:, None, :] * w.astype(np.float32)[None, :, :]   # exact in FP32
    for order in (slice(None), slice(None, None, -1)):
        acc = np.zeros((64, 32), np.float32)
        for k in range(2048)[order]:
            acc += prods[:, :, k]
        assert np.all(np.abs(acc.astype(np.float64) - exact) <= router.logit_error_bound(x, w))
