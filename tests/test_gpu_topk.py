"""Batched beam top-k (rq_topk) against the oracle, bit for bit: the indices and FP16 scores
of the k best candidates of every row in rank order (score descending, -0 below +0, equal
scores to the lower index).  Rows within one 16384-score segment, rows that run in two and
three stages (padded short tails included), ties, signed zeros, k at 1, n and 1024, rows not
a multiple of 8 long, and the two beam-search workloads at full size: 32 requests x 16 beams
x 512 codes keeping 16, and 32 requests x 512 beams x 512 codes keeping 512."""

import numpy as np
import pytest
import torch

import workloads
from oracle import topk as otopk
from tests.gpu_util import case, dev, host, require_gpu

pytestmark = pytest.mark.gpu


def _check(scores, k):
    rq = require_gpu()
    idx, vals = rq.topk(dev(scores), k)
    ref_i, ref_v = otopk.topk(scores, k)
    gi, gv = host(idx), host(vals)
    assert np.array_equal(gi, ref_i), "indices differ"
    assert np.array_equal(gv.view(np.uint16), ref_v.view(np.uint16)), "scores differ"


@pytest.mark.parametrize("rows,n,k,kind", [
    (3, 100, 7, "ties"), (4, 1001, 1000, "normal"), (2, 1001, 1, "ties"), (5, 16384, 16, "normal"),
    (2, 16385, 1024, "normal"), (3, 40000, 300, "ties"), (2, 200000, 64, "ties"), (1, 5000, 1024, "zeros"),
    (2, 1 << 20, 1024, "ties"), (7, 24, 24, "ties"),
])
def test_topk_parity(rows, n, k, kind):
    case("topk rows=%d n=%d k=%d %s" % (rows, n, k, kind))
    rng = np.random.default_rng(rows * n + k)
    if kind == "ties":
        s = rng.integers(-6, 6, size=(rows, n)).astype(np.float16)
    elif kind == "zeros":
        s = np.where(rng.random((rows, n)) < 0.5, np.float16(0.0), np.float16(-0.0)).astype(np.float16)
        s[:, ::97] = np.float16(-1.0)
    else:
        s = rng.standard_normal((rows, n)).astype(np.float16)
    _check(s, k)


@pytest.mark.slow
@pytest.mark.parametrize("beams,keep", [(16, 16), (512, 512)])
def test_beam_workloads_full_size(beams, keep):
    case("beam topk: 32 requests x %d beams x 512 codes, keep %d" % (beams, keep))
    s = workloads.beam_scores(np.random.default_rng(3000 + beams), 32, beams, 512)
    _check(s, keep)


def test_determinism_and_zero_rows():
    rq = require_gpu()
    case("topk determinism, rows = 0")
    s = dev(workloads.beam_scores(np.random.default_rng(5), 4, 64, 512))
    a, b = rq.topk(s, 200), rq.topk(s, 200)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    i, v = rq.topk(torch.zeros((0, 50), dtype=torch.float16, device="cuda"), 5)
    torch.cuda.synchronize()
    assert i.shape == (0, 5) and v.shape == (0, 5)


def test_argument_errors():
    rq = require_gpu()
    case("topk argument errors")
    s = torch.zeros((2, 50), dtype=torch.float16, device="cuda")
    for k in (0, 51):
        with pytest.raises(rq.RqError):
            rq.topk(s, k)
    with pytest.raises(rq.RqError):
        rq.topk(torch.zeros((1, 5000), dtype=torch.float16, device="cuda"), 1025)
