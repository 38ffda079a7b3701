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


# Gated layout: the gate/up linear's output columns come in blocks of 32 alternating gate
# and up features (columns [64b, 64b+32) gate of features [32b, 32b+32), [64b+32, 64b+64)
# their up values), so a kernel producing a 64-column block holds both operands of 32
# features.  The weight rows of W_gu are reordered the same way; since a linear computes
# each output column from its own weight row, reordering rows reorders output columns.
GATE_BLOCK = 32


def gate_up_order(f):
    """Row (or column) order of the gated layout: index i of the gated layout holds row
    ``order[i]`` of ``[gate (f) | up (f)]``."""
    if f % GATE_BLOCK != 0:
        raise ValueError("f must be a multiple of %d" % GATE_BLOCK)
    order = []
    for b in range(f // GATE_BLOCK):
        order.extend(range(b * GATE_BLOCK, (b + 1) * GATE_BLOCK))          # gate rows
        order.extend(range(f + b * GATE_BLOCK, f + (b + 1) * GATE_BLOCK))  # up rows
    return np.array(order, dtype=np.int64)


def gate_silu(y16):
    """``h`` of an FP16 gate/up output in the gated layout: put the columns back in
    ``[gate | up]`` order and apply ``silu_mul``."""
    y16 = np.asarray(y16)
    f = y16.shape[1] // 2
    gu = np.empty_like(y16)
    gu[:, gate_up_order(f)] = y16
    return silu_mul(gu, f)
