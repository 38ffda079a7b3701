"""GPU short-context attention core vs the oracle (oracle.attention).

FP16 outputs must lie within the oracle's derived bound (FP32 scores and softmax, FP16
probabilities, FP32 weighted sums, FP16 rounding) of its float64 result, on every element:
ragged request lengths, head counts that leave idle wavefronts, peaked and flat softmaxes,
and the 4096-token attention workload (128 requests x 32 positions, 16 heads of 128).
"""

import numpy as np
import pytest

from oracle import attention
from tests.gpu_util import case, dev, host, require_gpu

pytestmark = pytest.mark.gpu


def _qkv(rng, requests, length, heads, qk_scale=1.0):
    hidden = heads * 128
    t = requests * length
    ch = np.exp(rng.normal(0.0, 0.5, size=2 * hidden))                        # per-channel magnitudes
    qk = rng.standard_normal((t, 2 * hidden)) * ch * qk_scale / np.sqrt(np.sqrt(128))
    v = rng.standard_normal((t, hidden))
    return np.concatenate([qk, v], axis=1).astype(np.float16)


def _check(x, requests, length, heads):
    rq = require_gpu()
    y = host(rq.attention_core(dev(x), requests, length, heads))
    ref = attention.attention(x, requests, length, heads)
    tol = attention.tolerance(x, requests, length, heads, ref)
    d = np.abs(y.astype(np.float64) - ref.astype(np.float64))
    assert np.all(d <= tol), "max |d|/tol = %.3f" % float(np.max(d / tol))


@pytest.mark.parametrize("requests,length,heads,qk_scale", [
    (3, 1, 2, 1.0), (5, 17, 4, 1.0), (7, 32, 1, 1.0), (10, 8, 3, 3.0), (6, 32, 16, 0.0), (9, 31, 5, 6.0),
])
def test_attention_small(requests, length, heads, qk_scale):
    case("attention r=%d L=%d H=%d scale=%.1f" % (requests, length, heads, qk_scale))
    rng = np.random.default_rng(requests * 100 + length + heads)
    _check(_qkv(rng, requests, length, heads, qk_scale), requests, length, heads)


def test_attention_workload():
    """The attention workload's shape: 4096 tokens = 128 requests x 32 positions, 16 heads."""
    case("attention 128 x 32 x 16 heads")
    rng = np.random.default_rng(2002)
    _check(_qkv(rng, 128, 32, 16), 128, 32, 16)


def test_shape_errors():
    rq = require_gpu()
    case("attention argument errors")
    with pytest.raises(rq.RqError):
        rq.attention_core(dev(np.zeros((33, 384), np.float16)), 1, 33, 1)                 # length > 32
    with pytest.raises(rq.RqError):
        rq.attention_core(dev(np.zeros((4, 192), np.float16)), 1, 4, 1, head_dim=64)      # head_dim != 128
