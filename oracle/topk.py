"""Batched top-k selection over FP16 candidate rows (beam search).  Test infrastructure.

Page "FP8量化在生成式推荐系统OneRec-V2中的优化实践", §3.2, replaces the default TopK with
a RadixSelect kernel that runs batched with zero copies; its §5.3 keeps TopK results in FP16.
The beam search of OneRec serving keeps the best candidates of every request at each decoding
step; the page digesting the OneRec technical report (arXiv 2506.13695), in its paragraph on
training and inference optimizations, gives OneRec v1 serving a beam size of 512.

What is computed, for each row of ``n`` FP16 scores and a count ``1 <= k <= n``:

* candidates are ranked by score, larger first, in the IEEE-754 total order restricted to
  FP16 non-NaN values (so -0 ranks just below +0); equal scores rank the lower index first;
* the result is the first ``k`` candidates of that ranking: their indices (int) and their
  FP16 scores, in rank order.

The ranking is unique, so the result is exactly defined.  ``order_key`` maps an FP16 bit
pattern to an unsigned 16-bit key whose integer order is that total order (the plainest
encoding: flip every bit of a negative value, set the sign bit of a non-negative one); NaN
inputs are outside the contract.
"""

import numpy as np


def order_key(bits16):
    """Unsigned key of FP16 bit patterns whose integer order is the score order."""
    b = np.asarray(bits16, dtype=np.uint16).astype(np.uint32)
    neg = (b & 0x8000) != 0
    return np.where(neg, (~b) & 0xFFFF, b | 0x8000).astype(np.uint32)


def from_key(key):
    """Inverse of ``order_key``: FP16 bit patterns."""
    k = np.asarray(key, dtype=np.uint32)
    pos = (k & 0x8000) != 0
    return np.where(pos, k & 0x7FFF, (~k) & 0xFFFF).astype(np.uint16)


def topk(scores, k):
    """``(idx int64 [rows, k], vals FP16 [rows, k])`` of FP16 ``scores`` [rows, n]."""
    s = np.asarray(scores, dtype=np.float16)
    if s.ndim != 2:
        raise ValueError("scores must be [rows, n]")
    rows, n = s.shape
    if not 1 <= k <= n:
        raise ValueError("need 1 <= k <= n")
    if np.isnan(s).any():
        raise ValueError("NaN scores are outside the contract")
    keys = order_key(s.view(np.uint16)).astype(np.int64)
    idx = np.empty((rows, k), dtype=np.int64)
    for r in range(rows):
        # primary: key descending; secondary: index ascending (lexsort sorts by the last key first)
        order = np.lexsort((np.arange(n), -keys[r]))
        idx[r] = order[:k]
    vals = np.take_along_axis(s, idx, axis=1)
    return idx, vals
