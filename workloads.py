"""Seeded synthetic inputs for the W8A8 FP8 linear workloads.

This module only draws random FP16 tensors and routing decisions.  It holds none of
the method's arithmetic (no quantization, no GEMM, no SiLU) and is the one module that
both the oracle-based tests and the HIP path read their inputs from.

The pages measure on production OneRec-V2 traffic, which is not available; these
synthetic workloads stand in for it.  Their shapes follow the serving regime the pages
describe: short contexts of under 32 positions per request (page "FP8量化在生成式推荐
系统OneRec-V2中的优化实践", §3.2), batch 32 (§4.1), a merged QKV projection (§3.2),
and a fat-MoE decoder (page "Quantized Inference for OneRec-V2：生成式推荐开始直接吃
LLM 量化栈", section 关键证据).

Workloads (hidden 2048 unless stated):

1. ``dense_small``  X [64 x 512] with 1% outliers x20; W [512 x 512] ~ N(0, 0.02).
2. ``attention``    X and the attention output [4096 x 2048], N(0,1) times a per-channel
                    LogNormal(0, 0.5) magnitude; W_qkv [6144 x 2048]; W_o [2048 x 2048].
3. ``ffn``          X [4096 x 2048] as (1); W_gu [16384 x 2048] (gate rows then up rows);
                    W_dn [2048 x 8192].
4. ``moe``          X [16384 x 2048] as (1); top-2 of 32 experts with Zipf(1.1) loads and
                    one expert empty; W_gu [32 x 8192 x 2048]; W_dn [32 x 2048 x 4096].
5. ``layer_small_m`` 512 rows (32 requests x 16 beam rows), one layer's QKV, O, dense FFN
                    (8192) and MoE (4096) weights; activations Student-t(3) / sqrt(3).

Determinism: numpy PCG64, base seed ``1000 + workload number``, one child stream per
tensor from ``SeedSequence(seed).spawn`` in the order listed.  Draws are float32 and are
rounded to FP16 once.
"""

import numpy as np

HIDDEN = 2048

WORKLOADS = {
    1: "dense_small",
    2: "attention",
    3: "ffn",
    4: "moe",
    5: "layer_small_m",
}


# ----------------------------------------------------------------------------- draws

def _normal(rng, shape, std=1.0):
    return rng.standard_normal(shape, dtype=np.float32) * np.float32(std)


def acts_outliers(rng, m, k):
    """N(0,1) with 1% of the entries multiplied by 20."""
    z = rng.standard_normal((m, k), dtype=np.float32)
    b = rng.random((m, k), dtype=np.float32) < 0.01
    return (z * np.where(b, np.float32(20.0), np.float32(1.0))).astype(np.float16)


def acts_channel_lognormal(rng, m, k):
    """N(0,1) times a per-channel LogNormal(0, 0.5) magnitude."""
    c = rng.lognormal(0.0, 0.5, size=k).astype(np.float32)
    z = rng.standard_normal((m, k), dtype=np.float32)
    return (z * c[None, :]).astype(np.float16)


def acts_student_t(rng, m, k, nu=3.0):
    """Student-t(nu) scaled to unit standard deviation (heavy tails stress the amax)."""
    t = rng.standard_t(nu, size=(m, k))
    return (t / np.sqrt(nu / (nu - 2.0))).astype(np.float16)


def weights(rng, shape, std=0.02):
    """N(0, std^2) FP16 weights, drawn one leading slice at a time to bound memory."""
    out = np.empty(shape, dtype=np.float16)
    if len(shape) == 3:
        for e in range(shape[0]):
            out[e] = _normal(rng, shape[1:], std).astype(np.float16)
    else:
        out[...] = _normal(rng, shape, std).astype(np.float16)
    return out


def zipf_routing(rng, tokens, experts, top_k=2, alpha=1.1, empty_last=True):
    """Top-k expert ids with Zipf-skewed loads and FP16 routing weights.

    Rank r (1-based) has probability proportional to r^-alpha; the last rank gets
    probability 0 so that at least one expert is empty.  k distinct experts per token
    are drawn without replacement (Gumbel top-k), ranks are mapped to expert ids
    through a seeded permutation, and the weights are a softmax over k N(0,1) logits.
    """
    ranks = np.arange(1, experts + 1, dtype=np.float64)
    p = ranks ** (-alpha)
    if empty_last and experts > top_k:
        p[-1] = 0.0
    p /= p.sum()
    with np.errstate(divide="ignore"):
        logp = np.log(p)
    g = rng.gumbel(size=(tokens, experts))
    keys = logp[None, :] + g
    top = np.argsort(-keys, axis=1, kind="stable")[:, :top_k]
    rank_to_expert = rng.permutation(experts)
    ids = rank_to_expert[top].astype(np.int32)
    logits = rng.standard_normal((tokens, top_k))
    ex = np.exp(logits - logits.max(axis=1, keepdims=True))
    w = (ex / ex.sum(axis=1, keepdims=True)).astype(np.float16)
    return ids, w


# ------------------------------------------------------------------------- workloads

def beam_scores(rng, requests, beams, codes):
    """Beam-search candidate scores [requests, beams * codes] FP16: each beam's running
    log-probability (sorted, the best beam first) plus a log-softmax over ``codes`` next
    semantic-ID codes, as a decoding step of a generative recommender produces them."""
    running = -np.sort(rng.exponential(3.0, size=(requests, beams)), axis=1)
    logits = rng.standard_normal((requests, beams, codes)) * 2.0
    m = logits.max(axis=2, keepdims=True)
    logp = logits - m - np.log(np.exp(logits - m).sum(axis=2, keepdims=True))
    return (running[:, :, None] + logp).reshape(requests, beams * codes).astype(np.float16)


def _streams(seed, n):
    return [np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(n)]


def make(workload, seed=None, **size):
    """Inputs of one workload as a dict of numpy arrays.

    ``size`` overrides the dimensions (``m``, ``k``, ``n``, ``f``, ``t``, ``e``,
    ``top_k``) so that parity tests can draw the same recipe at sizes the oracle
    finishes in seconds.
    """
    w = int(workload)
    seed = 1000 + w if seed is None else int(seed)
    if w == 1:
        m, k, n = size.get("m", 64), size.get("k", 512), size.get("n", 512)
        r = _streams(seed, 2)
        return {"x": acts_outliers(r[0], m, k), "w": weights(r[1], (n, k))}
    if w == 2:
        m, k = size.get("m", 4096), size.get("k", HIDDEN)
        nq, no = size.get("n_qkv", 3 * k), size.get("n_o", k)
        r = _streams(seed, 4)
        return {"x": acts_channel_lognormal(r[0], m, k),
                "attn_out": acts_channel_lognormal(r[1], m, no),
                "w_qkv": weights(r[2], (nq, k)),
                "w_o": weights(r[3], (k, no))}
    if w == 3:
        m, k, f = size.get("m", 4096), size.get("k", HIDDEN), size.get("f", 8192)
        r = _streams(seed, 3)
        return {"x": acts_outliers(r[0], m, k),
                "w_gu": weights(r[1], (2 * f, k)),
                "w_dn": weights(r[2], (k, f))}
    if w == 4:
        t, k, f = size.get("t", 16384), size.get("k", HIDDEN), size.get("f", 4096)
        e, top_k = size.get("e", 32), size.get("top_k", 2)
        r = _streams(seed, 4)
        x = acts_outliers(r[0], t, k)
        ids, tw = zipf_routing(r[1], t, e, top_k)
        return {"x": x, "ids": ids, "topk_w": tw,
                "w_gu": weights(r[2], (e, 2 * f, k)),
                "w_dn": weights(r[3], (e, k, f))}
    if w == 5:
        m, k = size.get("m", 512), size.get("k", HIDDEN)
        f, fe = size.get("f", 8192), size.get("f_moe", 4096)
        e, top_k = size.get("e", 32), size.get("top_k", 2)
        r = _streams(seed, 11)
        out = {"x_qkv": acts_student_t(r[0], m, k),
               "x_o": acts_student_t(r[1], m, k),
               "x_ffn": acts_student_t(r[2], m, k),
               "x_moe": acts_student_t(r[3], m, k)}
        ids, tw = zipf_routing(r[4], m, e, top_k)
        out.update({"ids": ids, "topk_w": tw,
                    "w_qkv": weights(r[5], (3 * k, k)),
                    "w_o": weights(r[6], (k, k)),
                    "w_gu": weights(r[7], (2 * f, k)),
                    "w_dn": weights(r[8], (k, f)),
                    "w_gu_moe": weights(r[9], (e, 2 * fe, k)),
                    "w_dn_moe": weights(r[10], (e, k, fe))})
        return out
    raise ValueError("unknown workload %r" % (workload,))


def gemm_shapes(workload, **size):
    """The (M, N, K) triples of the workload's linears, MoE counted over routed rows."""
    w = int(workload)
    if w == 1:
        return [(size.get("m", 64), size.get("n", 512), size.get("k", 512))]
    if w == 2:
        m, k = size.get("m", 4096), size.get("k", HIDDEN)
        return [(m, 3 * k, k), (m, k, k)]
    if w == 3:
        m, k, f = size.get("m", 4096), size.get("k", HIDDEN), size.get("f", 8192)
        return [(m, 2 * f, k), (m, k, f)]
    if w == 4:
        t, k, f = size.get("t", 16384), size.get("k", HIDDEN), size.get("f", 4096)
        r = t * size.get("top_k", 2)
        return [(r, 2 * f, k), (r, k, f)]
    if w == 5:
        m, k = size.get("m", 512), size.get("k", HIDDEN)
        f, fe = size.get("f", 8192), size.get("f_moe", 4096)
        r = m * size.get("top_k", 2)
        return [(m, 3 * k, k), (m, k, k), (m, 2 * f, k), (m, k, f), (r, 2 * fe, k), (r, k, fe)]
    raise ValueError("unknown workload %r" % (workload,))


def gemm_flops(workload, **size):
    return sum(2 * m * n * k for (m, n, k) in gemm_shapes(workload, **size))
