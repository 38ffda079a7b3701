"""MoE router: FP16 gate logits and top-k expert selection.  Test infrastructure.

Page "FP8量化在生成式推荐系统OneRec-V2中的优化实践", §2.1, keeps the routing gate in FP16
(it is not quantized); the step before the MoE grouped GEMM turns each token's gate logits
into the ids of its top-k experts and their combine weights.  The pages give no formula for
the weights; the reading taken here is the common one for top-k routing: the softmax of the
selected logits (equal to the full softmax's top-k probabilities renormalized to sum 1).

Definitions, for a token row x [K] and gate weights W [E x K], both FP16:

1. ``logit[e] = sum_k x[k] * W[e, k]`` - computed here in float64 (each FP16 x FP16 product
   is exact; the float64 sum of K <= 8192 of them is within K * 2^-53 of the real sum).
2. Selection: the top_k experts by logit, larger first; equal logits go to the lower expert
   index (a total order, so the result is unique).
3. Weights: ``w_i = exp(l_i - l_0) / sum_j exp(l_j - l_0)`` over the selected logits (l_0 the
   largest), rounded once to FP16.
"""

import numpy as np


def logits(x16, w16):
    """float64 gate logits [T, E] of FP16 rows x [T, K] and gate weights W [E, K]."""
    x = np.asarray(x16, dtype=np.float16).astype(np.float64)
    w = np.asarray(w16, dtype=np.float16).astype(np.float64)
    if x.shape[1] != w.shape[1]:
        raise ValueError("K mismatch")
    return x @ w.T


def select(lg, top_k):
    """Top-k expert ids per row of logits [T, E] (larger first, ties to the lower index)."""
    lg = np.asarray(lg, dtype=np.float64)
    t, e = lg.shape
    if not 1 <= top_k <= e:
        raise ValueError("top_k out of range")
    idx = np.arange(e)
    ids = np.empty((t, top_k), dtype=np.int32)
    for r in range(t):
        order = sorted(idx, key=lambda j: (-lg[r, j], j))
        ids[r] = order[:top_k]
    return ids


def weights(lg, ids):
    """FP16 softmax of the selected logits, per row (float64, one rounding)."""
    lg = np.asarray(lg, dtype=np.float64)
    sel = np.take_along_axis(lg, np.asarray(ids, dtype=np.int64), axis=1)
    z = np.exp(sel - sel[:, :1])
    return (z / z.sum(axis=1, keepdims=True)).astype(np.float16)


def route(x16, w16, top_k):
    """``(ids [T, top_k] int32, weights [T, top_k] FP16, logits [T, E] float64)``."""
    lg = logits(x16, w16)
    ids = select(lg, top_k)
    return ids, weights(lg, ids), lg


def logit_error_bound(x16, w16):
    """Bound on |FP32-accumulated logit - exact logit|: the products are exact in FP32, and
    any order of K FP32 additions errs by at most gamma_K * sum |x w|, gamma_K = K u / (1 - K u),
    u = 2^-24."""
    x = np.abs(np.asarray(x16, dtype=np.float16).astype(np.float64))
    w = np.abs(np.asarray(w16, dtype=np.float16).astype(np.float64))
    k = x.shape[1]
    u = 2.0 ** -24
    return (k * u / (1 - k * u)) * (x @ w.T)
