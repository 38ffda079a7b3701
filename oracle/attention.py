"""Short-context attention core between the QKV and O projections.  Test infrastructure.

Page "FP8量化在生成式推荐系统OneRec-V2中的优化实践", §3.2, describes the serving context as
short sequences (tens of positions per request); page "Quantized Inference for OneRec-V2：
生成式推荐开始直接吃 LLM 量化栈", section 关键证据, quantizes only the q/k/v/o linears, so the
attention core between them stays FP16.  The pages give no head layout, mask or scaling;
the readings taken here (plain ones, consistent with the 2048-wide hidden state):

* the QKV projection's output row is [q (hidden) | k (hidden) | v (hidden)] (the merged
  [Wq; Wk; Wv] linear), each split into H heads of D = hidden / H contiguous columns
  (H = 16, D = 128 for the 2048-wide workload);
* requests are independent and hold L consecutive token rows (L <= 32); position i of a
  request attends to positions j <= i of the same request (causal, generative decoding);
* scores are q . k / sqrt(D); the softmax is over the allowed positions; the output row is
  [head 0 | head 1 | ...], the O projection's input.

The oracle computes every step in float64 from the FP16 inputs and rounds the output once
to FP16.  ``tolerance`` bounds a GPU result that forms the scores with FP32 accumulation,
the softmax in FP32 and the probability-weighted sum with FP16 probabilities and FP32
accumulation.
"""

import numpy as np


def _split(qkv16, requests, length, heads):
    x = np.asarray(qkv16, dtype=np.float16).astype(np.float64)
    t, width = x.shape
    if t != requests * length or width % 3:
        raise ValueError("qkv must be [requests * length, 3 * hidden]")
    hidden = width // 3
    if hidden % heads:
        raise ValueError("hidden not divisible by heads")
    d = hidden // heads
    shape = (requests, length, heads, d)
    q = x[:, :hidden].reshape(shape)
    k = x[:, hidden:2 * hidden].reshape(shape)
    v = x[:, 2 * hidden:].reshape(shape)
    return q, k, v, d


def probabilities(qkv16, requests, length, heads):
    """float64 attention probabilities [requests, heads, L (query), L (key)] and scores."""
    q, k, _, d = _split(qkv16, requests, length, heads)
    s = np.einsum("rihd,rjhd->rhij", q, k) / np.sqrt(d)
    allowed = np.tril(np.ones((length, length), dtype=bool))
    s = np.where(allowed, s, -np.inf)
    p = np.exp(s - s.max(axis=-1, keepdims=True))
    return p / p.sum(axis=-1, keepdims=True), s


def attention(qkv16, requests, length, heads):
    """FP16 attention output [requests * L, hidden]."""
    _, _, v, d = _split(qkv16, requests, length, heads)
    p, _ = probabilities(qkv16, requests, length, heads)
    o = np.einsum("rhij,rjhd->rihd", p, v)
    return o.reshape(requests * length, heads * d).astype(np.float16)


def tolerance(qkv16, requests, length, heads, y_ref):
    """Per-element bound on |y_gpu - y_ref|.

    With u = 2^-24: a score accumulated in FP32 over D exact FP16 products and scaled by an
    FP32 1/sqrt(D) errs by at most ds = (gamma_D + 2u) * sum_k |q_k k_k| / sqrt(D); the FP32
    softmax then turns it into a relative error of at most 2 ds + 2^-20 per probability
    (exp within a few FP32 ulps, one division); rounding a probability to FP16 adds 2^-11
    and the FP32 sum over L terms gamma_L.  So

        |o - o*| <= (2^-11 + 2 ds_max + 2^-20 + gamma_L) * sum_j p_j |v_j|,

    doubled for margin, plus 2 FP16 ulps of the final rounding."""
    q, k, v, d = _split(qkv16, requests, length, heads)
    p, _ = probabilities(qkv16, requests, length, heads)
    u = 2.0 ** -24
    gamma = lambda n: n * u / (1 - n * u)  # noqa: E731
    abs_s = np.einsum("rihd,rjhd->rhij", np.abs(q), np.abs(k)) / np.sqrt(d)
    ds = (gamma(d) + 2 * u) * abs_s.max(axis=-1)                    # [r, h, i]
    rel = 2.0 ** -11 + 2 * ds + 2.0 ** -20 + gamma(length)
    weight = np.einsum("rhij,rjhd->rihd", p, np.abs(v))              # sum_j p_j |v_j|
    bound = 2 * rel.transpose(0, 2, 1)[..., None] * weight
    from .linear import ulp16
    return bound.reshape(requests * length, heads * d) + 2 * ulp16(y_ref)
