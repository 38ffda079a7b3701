"""FFN intermediate ``h = fl16(silu(g) * u)``.  Test infrastructure.

The pages quantize the dense FFN linears and the expert linears (page "Quantized
Inference for OneRec-V2：生成式推荐开始直接吃 LLM 量化栈", section 关键证据) and
cast every linear's output back to FP16 before the next layer.  They do not name the
activation; the workload uses SiLU(gate) * up, so the FFN runs as

    g|u = linear(X, W_gu)        W_gu rows [0, F) are the gate, rows [F, 2F) the up channels
    h   = fl16(silu(g) * u)      silu(g) = g / (1 + exp(-g)), evaluated once in float64
    y   = linear(quantize_rows(h), W_dn)

so ``h`` is an FP16 tensor that the row quantizer re-quantizes per token.
"""

import numpy as np


def silu_mul(gu, f):
    """``fl16(g * u / (1 + exp(-g)))`` for FP16 rows laid out as ``[g (f) | u (f)]``."""
    gu16 = np.asarray(gu)
    if gu16.dtype != np.float16 or gu16.ndim != 2 or gu16.shape[1] != 2 * f:
        raise ValueError("expected FP16 rows of width 2*f")
    g = gu16[:, :f].astype(np.float64)
    u = gu16[:, f:].astype(np.float64)
    with np.errstate(over="ignore"):
        h = g * u / (1.0 + np.exp(-g))
        return h.astype(np.float16)
