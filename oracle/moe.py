"""Sparse-MoE expert grouped linear: routing plan, per-expert W8A8 linear, combine.

Test infrastructure.  Page "Quantized Inference for OneRec-V2：生成式推荐开始直接吃 LLM
量化栈", section 关键证据, puts the MoE grouped GEMM on the quantized path; page
"FP8量化在生成式推荐系统OneRec-V2中的优化实践", §2.1, keeps the routing gate in FP16,
so the gate's top-k expert ids and FP16 weights arrive here as data.

Routing plan (integers):

1. slot ``j = t * top_k + k`` of token ``t`` goes to expert ``e = ids[t, k]``;
2. ``counts[e]`` = number of slots on expert e; ``offsets`` = exclusive prefix sum, E + 1 entries;
3. canonical permuted order: slots sorted by ``(e, j)`` ascending, i.e. a stable
   counting sort by expert; ``perm[r]`` is the slot in permuted row r and ``pos[j]`` the
   row holding slot j.

Grouped linear: permuted row r of expert e multiplies its input row by ``W[e]`` with that
expert's per-channel scales (``oracle.linear``).  With ``in_layout == TOKENS`` the input
row is token ``perm[r] // top_k`` (quantized once per token, before dispatch); with
``PERMUTED`` it is row r of an already permuted input.  With ``act == SILU_MUL`` each
input row is ``[g | u]`` and ``oracle.ffn.silu_mul`` makes the FP16 row that is quantized.

Combine (``out_layout == COMBINED``):
``out[t] = fl16(sum_k w[t, k] * y[pos[t * top_k + k]])`` over the FP16 permuted outputs,
summed in float64 and rounded once.
"""

import numpy as np

from . import ffn, linear, quant, wscale

IN_TOKENS, IN_PERMUTED = 0, 1
OUT_PERMUTED, OUT_COMBINED = 0, 1
ACT_NONE, ACT_SILU_MUL = 0, 1


def plan(ids, num_experts):
    """Return ``(counts [E], offsets [E+1], perm [R], pos [R])`` as int64 arrays."""
    ids = np.asarray(ids)
    flat = ids.reshape(-1).astype(np.int64)
    if flat.size and (flat.min() < 0 or flat.max() >= num_experts):
        raise ValueError("expert id out of range")
    counts = np.zeros(num_experts, dtype=np.int64)
    for e in flat:
        counts[e] += 1
    offsets = np.zeros(num_experts + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    perm = np.empty(flat.size, dtype=np.int64)
    fill = offsets[:-1].copy()
    for j, e in enumerate(flat):          # ascending j: stable within each expert
        perm[fill[e]] = j
        fill[e] += 1
    pos = np.empty(flat.size, dtype=np.int64)
    pos[perm] = np.arange(flat.size, dtype=np.int64)
    return counts, offsets, perm, pos


def grouped_linear(x, in_layout, act, ids, w_q, s_w, out_layout=OUT_PERMUTED, topk_w=None,
                   gran=wscale.CHANNEL, a_fmt="e4m3"):
    """Oracle of one grouped call.

    ``x`` FP16 [T or R, K or 2K]; ``ids`` int [T, top_k]; ``w_q`` uint8 [E, N, K];
    ``s_w`` float32 [E, N] (or per expert the layout of ``gran``, see ``oracle.wscale``);
    ``topk_w`` FP16 [T, top_k] for the combined output.

    Returns a dict with ``y`` (FP16 [R, N] permuted or [T, N] combined), ``y_perm``
    (FP16 [R, N]), ``a_q``/``a_scale`` (the quantized GEMM input: T rows for TOKENS, R
    rows for PERMUTED), ``h`` (FP16 SiLU rows or None) and the plan.
    """
    ids = np.asarray(ids)
    t, top_k = ids.shape
    e_count, n, k = w_q.shape
    r_total = t * top_k
    counts, offsets, perm, pos = plan(ids, e_count)

    x16 = np.asarray(x, dtype=np.float16)
    expect_rows = t if in_layout == IN_TOKENS else r_total
    width = 2 * k if act == ACT_SILU_MUL else k
    if x16.shape != (expect_rows, width):
        raise ValueError("input shape %r, expected %r" % (x16.shape, (expect_rows, width)))

    h = ffn.silu_mul(x16, k) if act == ACT_SILU_MUL else None
    rows = h if h is not None else x16
    a_q, a_scale = quant.quantize_rows(rows, a_fmt)

    y_perm = np.zeros((r_total, n), dtype=np.float16)
    for e in range(e_count):
        lo, hi = offsets[e], offsets[e + 1]
        if hi == lo:
            continue
        r = np.arange(lo, hi)
        src = perm[r] // top_k if in_layout == IN_TOKENS else r
        if gran == wscale.CHANNEL:
            y_perm[r] = linear.linear(a_q[src], a_scale[src], w_q[e], s_w[e], a_fmt)
        else:
            y_perm[r] = wscale.linear(a_q[src], a_scale[src], w_q[e], s_w[e], gran, a_fmt)

    out = {"y_perm": y_perm, "a_q": a_q, "a_scale": a_scale, "h": h,
           "counts": counts, "offsets": offsets, "perm": perm, "pos": pos}
    if out_layout == OUT_COMBINED:
        out["y"] = combine(y_perm, pos, topk_w)
    else:
        out["y"] = y_perm
    return out


def combine(y_perm, pos, topk_w):
    """``fl16(sum_k w[t, k] * y_perm[pos[t*top_k + k]])`` in float64."""
    w = np.asarray(topk_w, dtype=np.float16).astype(np.float64)
    t, top_k = w.shape
    yp = np.asarray(y_perm, dtype=np.float16).astype(np.float64)
    acc = np.zeros((t, yp.shape[1]), dtype=np.float64)
    for slot in range(top_k):
        acc += w[:, slot][:, None] * yp[pos[np.arange(t) * top_k + slot]]
    return acc.astype(np.float16)


def grouped_linear_check(y_gpu_perm, a_q, a_scale, in_layout, ids, w_q, s_w, gran=wscale.CHANNEL,
                         a_fmt="e4m3"):
    """Stage check of a GPU permuted GEMM output against the GPU's own quantized input.

    Returns ``(ok, worst |d|/tol)`` over all permuted rows.
    """
    t, top_k = np.asarray(ids).shape
    counts, offsets, perm, _ = plan(ids, w_q.shape[0])
    worst, ok = 0.0, True
    for e in range(w_q.shape[0]):
        lo, hi = offsets[e], offsets[e + 1]
        if hi == lo:
            continue
        r = np.arange(lo, hi)
        src = perm[r] // top_k if in_layout == IN_TOKENS else r
        if gran == wscale.CHANNEL:
            good, ratio, _ = linear.check(y_gpu_perm[r], a_q[src], a_scale[src], w_q[e], s_w[e], a_fmt)
        else:
            good, ratio, _ = wscale.check(y_gpu_perm[r], a_q[src], a_scale[src], w_q[e], s_w[e], gran, a_fmt)
        ok &= good
        worst = max(worst, ratio)
    return ok, worst
