"""Weight-scale granularities: per output channel, per tensor, per 128 x 128 block.

Test infrastructure.  Page "FP8量化在生成式推荐系统OneRec-V2中的优化实践", §2.1 and §2.2,
gives each kind of weight its own scale granularity: the attention projections one scale
per output channel, the dense FFN weights one scale for the whole tensor, and the MoE
expert weights one scale per block of 128 output channels x 128 input channels.  Page
"Quantized Inference for OneRec-V2：生成式推荐开始直接吃 LLM 量化栈", section 关键证据, uses
per-channel weights throughout; that is the default everywhere else in this oracle.

Every granularity quantizes with the row quantizer's formula (``oracle.quant``) applied
to the set of values that shares a scale:

    amax = max |w| over the set,  s = fl32(max(amax, 2^-24) / 448),  q = E4M3(fl32(w / s)).

Scale layouts for a weight matrix [N x K]: CHANNEL ``[N]``, TENSOR ``[1]``, BLOCK128
``[N / 128, K / 128]`` (block (i, j) covers rows 128 i .. 128 i + 127 and columns
128 j .. 128 j + 127).  Block scales need N and K to be multiples of 128: the pages' blocks
tile the matrix and every weight shape of the workloads is such a multiple.

Linear with block scales.  With A the quantized activations and s_x their per-token
scales, the output is

    y*[m, n] = s_x[m] * sum_j S[n // 128, j] * P_j[m, n],
    P_j[m, n] = sum_{k in block j} dec(a_q[m, k]) * dec(w_q[n, k]),

each K block's partial product scaled by its block scale and the scaled partials summed:
the "FP32 accumulate per block, then scale" structure of block-wise FP8 GEMMs.  P_j is
exact (see ``oracle.linear``); y* is formed in float64 and rounded once to FP16.  The
tolerance generalizes the per-channel one term by term:

    |y - fl16(y*)| <= 2 ulp16 + 1e-3 * s_x[m] * sum_j S[n // 128, j] * sum_{k in j} |dec(a) dec(w)|.
"""

import numpy as np

from . import e4m3
from . import linear as lin
from . import quant

CHANNEL, TENSOR, BLOCK128 = 0, 1, 2
BLOCK = 128


def _check_fp16_2d(w):
    w16 = np.asarray(w)
    if w16.dtype != np.float16 or w16.ndim != 2:
        raise TypeError("expected a 2-D FP16 weight matrix")
    return w16


def quantize_tensor(w):
    """One scale for the whole matrix.  Returns ``(q [N, K] uint8, s [1] float32)``."""
    w16 = _check_fp16_2d(w)
    wd = w16.astype(np.float64)
    amax = np.max(np.abs(wd)) if wd.size else 0.0
    s = quant.row_scale(np.array([amax]))
    quotient = (wd / np.float64(s[0])).astype(np.float32)
    return e4m3.encode(quotient.astype(np.float64)), s


def quantize_blocks(w):
    """One scale per 128 x 128 block.  Returns ``(q [N, K] uint8, s [N/128, K/128] float32)``."""
    w16 = _check_fp16_2d(w)
    n, k = w16.shape
    if n % BLOCK or k % BLOCK:
        raise ValueError("block scales need N and K to be multiples of %d" % BLOCK)
    wd = w16.astype(np.float64)
    nb, kb = n // BLOCK, k // BLOCK
    blocks = np.abs(wd).reshape(nb, BLOCK, kb, BLOCK)
    amax = blocks.max(axis=(1, 3)) if wd.size else np.zeros((nb, kb))
    s = quant.row_scale(amax)
    s_full = np.repeat(np.repeat(s.astype(np.float64), BLOCK, axis=0), BLOCK, axis=1)
    quotient = (wd / s_full).astype(np.float32)
    return e4m3.encode(quotient.astype(np.float64)), s


def quantize(w, gran):
    """Quantize a weight matrix at granularity ``gran``; returns ``(q, s)``."""
    if gran == CHANNEL:
        return quant.quantize_rows(w)
    if gran == TENSOR:
        return quantize_tensor(w)
    if gran == BLOCK128:
        return quantize_blocks(w)
    raise ValueError("unknown granularity %r" % (gran,))


def _k_blocks(k):
    return [(j, slice(j * BLOCK, (j + 1) * BLOCK)) for j in range(k // BLOCK)]


def _reference(x_q, s_x, w_q, w_s, gran, a_fmt="e4m3"):
    """(float64 y*, float64 tolerance weight sum_j S |P|_j) for each output."""
    sx = np.asarray(s_x, dtype=np.float64)[:, None]
    if gran == CHANNEL or gran == TENSOR:
        n = w_q.shape[0]
        sw = np.asarray(w_s, dtype=np.float64).reshape(-1)
        sw = np.full(n, sw[0]) if gran == TENSOR else sw
        acc = lin.gemm_exact(x_q, w_q, a_fmt)
        absacc = lin.gemm_abs_exact(x_q, w_q, a_fmt)
        return acc * sx * sw[None, :], absacc * sw[None, :]
    if gran != BLOCK128:
        raise ValueError("unknown granularity %r" % (gran,))
    n, k = w_q.shape
    if n % BLOCK or k % BLOCK:
        raise ValueError("block scales need N and K to be multiples of %d" % BLOCK)
    S = np.asarray(w_s, dtype=np.float64).reshape(n // BLOCK, k // BLOCK)
    total = np.zeros((x_q.shape[0], n))
    weight = np.zeros((x_q.shape[0], n))
    for j, ks in _k_blocks(k):
        s_col = np.repeat(S[:, j], BLOCK)[None, :]          # block scale of each output column
        total += s_col * lin.gemm_exact(x_q[:, ks], w_q[:, ks], a_fmt)
        weight += s_col * lin.gemm_abs_exact(x_q[:, ks], w_q[:, ks], a_fmt)
    return total * sx, weight


def linear(x_q, s_x, w_q, w_s, gran, a_fmt="e4m3"):
    """FP16 output of the quantized linear with weight scales of granularity ``gran``."""
    y, _ = _reference(x_q, s_x, w_q, w_s, gran, a_fmt)
    return y.astype(np.float16)


def check(y_gpu, x_q, s_x, w_q, w_s, gran, a_fmt="e4m3"):
    """Compare a GPU output with the oracle.  Returns ``(ok, worst |d|/tol, y_ref)``."""
    y, weight = _reference(x_q, s_x, w_q, w_s, gran, a_fmt)
    y_ref = y.astype(np.float16)
    tol = 2.0 * lin.ulp16(y_ref) + 1e-3 * np.asarray(s_x, dtype=np.float64)[:, None] * weight
    d = np.abs(np.asarray(y_gpu, dtype=np.float64) - y_ref.astype(np.float64))
    ratio = float(np.max(d / tol)) if d.size else 0.0
    return bool((d <= tol).all()), ratio, y_ref
