"""Pins of the oracle's short-context attention core (oracle.attention).

Closed forms (one position, uniform scores, a planted dominant key), structure (causality,
head independence) and a scalar-loop brute force; the tolerance admits an FP32 / FP16
simulation of the GPU's arithmetic and rejects a dropped mask or scale.
"""

import math

import numpy as np

from oracle import attention


def _qkv(rng, requests, length, heads, d, scale=1.0):
    return (rng.standard_normal((requests * length, 3 * heads * d)) * scale).astype(np.float16)


def test_single_position_returns_v():
    rng = np.random.default_rng(1)
    x = _qkv(rng, 5, 1, 4, 32)
    o = attention.attention(x, 5, 1, 4)
    assert np.array_equal(o, x[:, 2 * 128:])


def test_uniform_scores_give_causal_means():
    rng = np.random.default_rng(2)
    r, length, h, d = 2, 7, 2, 16
    x = _qkv(rng, r, length, h, d)
    x[:, :h * d] = 0                                          # q = 0: every allowed score is 0
    o = attention.attention(x, r, length, h)
    v = x[:, 2 * h * d:].astype(np.float64).reshape(r, length, h * d)
    ref = (np.cumsum(v, axis=1) / np.arange(1, length + 1)[None, :, None]).reshape(r * length, h * d)
    # averages of FP16 values often sit exactly on an FP16 rounding midpoint, where the
    # oracle's p-weighted sum (p = 1/(i+1) rounded) may fall on either side: 1 ulp apart
    d16 = np.abs(o.astype(np.float64) - ref)
    assert np.all(d16 <= np.spacing(np.abs(ref).astype(np.float16)).astype(np.float64))


def test_scalar_loop_brute_force():
    rng = np.random.default_rng(3)
    r, length, h, d = 2, 5, 3, 8
    x = _qkv(rng, r, length, h, d)
    o = attention.attention(x, r, length, h)
    xd = x.astype(np.float64)
    for b in range(r):
        for hh in range(h):
            for i in range(length):
                qi = xd[b * length + i, hh * d:(hh + 1) * d]
                s = []
                for j in range(i + 1):
                    kj = xd[b * length + j, h * d + hh * d:h * d + (hh + 1) * d]
                    s.append(sum(qi[t] * kj[t] for t in range(d)) / math.sqrt(d))
                m = max(s)
                e = [math.exp(v - m) for v in s]
                for c in range(d):
                    acc = sum(e[j] * xd[b * length + j, 2 * h * d + hh * d + c] for j in range(i + 1)) / sum(e)
                    assert abs(float(o[b * length + i, hh * d + c]) - acc) <= 2.0 ** -10 * max(abs(acc), 2.0 ** -14)


def test_causality_and_request_independence():
    rng = np.random.default_rng(4)
    r, length, h, d = 3, 8, 2, 16
    x = _qkv(rng, r, length, h, d)
    o = attention.attention(x, r, length, h)
    y = x.copy()
    y[length + 5:length + 8, h * d:] = rng.standard_normal((3, 2 * h * d)).astype(np.float16)  # later k, v of request 1
    o2 = attention.attention(y, r, length, h)
    assert np.array_equal(o[:length + 5], o2[:length + 5])                  # earlier rows unchanged
    assert np.array_equal(o[2 * length:], o2[2 * length:])                  # other requests unchanged
    assert not np.array_equal(o[length + 5:2 * length], o2[length + 5:2 * length])


def test_heads_are_independent_column_blocks():
    rng = np.random.default_rng(5)
    r, length, h, d = 2, 6, 4, 8
    x = _qkv(rng, r, length, h, d)
    perm = np.array([2, 0, 3, 1])
    cols = np.arange(h * d).reshape(h, d)[perm].reshape(-1)
    y = np.concatenate([x[:, :h * d][:, cols], x[:, h * d:2 * h * d][:, cols], x[:, 2 * h * d:][:, cols]], axis=1)
    assert np.array_equal(attention.attention(y, r, length, h), attention.attention(x, r, length, h)[:, cols])


def test_planted_dominant_key():
    rng = np.random.default_rng(6)
    r, length, h, d = 1, 4, 1, 64
    x = _qkv(rng, r, length, h, d, scale=0.01)
    x[3, :d] = 1.0                                            # query 3
    x[1, d:2 * d] = 1.0                                       # key 1 matches it: score 64 / 8 = 8
    o = attention.attention(x, r, length, h)
    assert np.all(np.abs(o[3].astype(np.float64) - x[1, 2 * d:].astype(np.float64)) < 2e-3)


def test_tolerance_admits_the_gpu_arithmetic_and_rejects_a_shift():
    rng = np.random.default_rng(7)
    r, length, h, d = 4, 32, 2, 128
    x = _qkv(rng, r, length, h, d)
    ref = attention.attention(x, r, length, h)
    tol = attention.tolerance(x, r, length, h, ref)
    # FP32 scores and softmax, FP16 probabilities, FP32 weighted sum: the GPU's arithmetic
    xf = x.astype(np.float32)
    q = xf[:, :h * d].reshape(r, length, h, d)
    k = xf[:, h * d:2 * h * d].reshape(r, length, h, d)
    v = xf[:, 2 * h * d:].reshape(r, length, h, d)
    s = np.einsum("rihd,rjhd->rhij", q, k).astype(np.float32) * np.float32(1 / math.sqrt(d))
    s = np.where(np.tril(np.ones((length, length), bool)), s, -np.inf).astype(np.float32)
    e = np.exp(s - s.max(-1, keepdims=True)).astype(np.float32)
    p16 = (e / e.sum(-1, keepdims=True)).astype(np.float16).astype(np.float32)
    sim = np.einsum("rhij,rjhd->rihd", p16, v).astype(np.float32).reshape(r * length, h * d).astype(np.float16)
    d_sim = np.abs(sim.astype(np.float64) - ref.astype(np.float64))
    assert np.all(d_sim <= tol)
    # plausible mistakes fall far outside it: a dropped causal mask, a dropped 1/sqrt(D)
    for mask, scale in ((np.ones((length, length), bool), 1 / math.sqrt(d)),
                        (np.tril(np.ones((length, length), bool)), 1.0)):
        sw = np.where(mask, np.einsum("rihd,rjhd->rhij", q, k) * scale, -np.inf)
        pw = np.exp(sw - sw.max(-1, keepdims=True))
        pw /= pw.sum(-1, keepdims=True)
        wrong = np.einsum("rhij,rjhd->rihd", pw, v).reshape(r * length, h * d).astype(np.float16)
        assert not np.all(np.abs(wrong.astype(np.float64) - ref.astype(np.float64)) <= tol)
