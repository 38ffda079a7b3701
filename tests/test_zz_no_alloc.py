"""The allocation-free linear (rq_fp8_linear_noalloc) against rq_fp8_linear, through the C ABI.

Both run the same quantizer and GEMM kernels, so the outputs must agree bit for bit (the
linear's own parity with the oracle is tested elsewhere).  Two calls in a row, the second
with a smaller input, check that the shared static buffer carries nothing from one call to
the next; no PyTorch allocation happens inside the calls.
"""

import ctypes

import numpy as np
import pytest
import torch

import workloads
from tests.gpu_util import case, dev, host, require_gpu

pytestmark = pytest.mark.gpu


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _reference(lib, x, m, k, act, wq, ws, n, y):
    # the workspace that lets rq_fp8_linear split K as the static buffer does
    need = lib.rq_fp8_linear_workspace_size_ex(m, n, k, act)
    wsp = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    st = lib.rq_fp8_linear(_p(x), m, k, act, _p(wq), _p(ws), n, _p(y), _p(wsp), wsp.numel(), None, _stream())
    assert st == 0, st
    torch.cuda.synchronize()


@pytest.mark.parametrize("act", [0, 1, 2])
def test_noalloc_matches_linear(act):
    rq = require_gpu()
    from fp8_quantized_generative_amd import _lib
    lib = _lib.load()
    # the larger call first, then smaller ones that reuse (part of) the same buffer: 512 rows
    # split K (partial sums in the buffer too), the ragged one does not
    for m, k, n, seed in ((2048, 2048, 2048, 1), (512, 8192, 2048, 3), (130, 528, 320, 2)):
        case("noalloc act=%d m=%d k=%d n=%d" % (act, m, k, n))
        rng = np.random.default_rng(seed + 10 * act)
        xw = 2 * k if act == 1 else k
        x = dev(workloads.acts_student_t(rng, m, xw))
        wq, ws = rq.quant_weights(dev(workloads.weights(rng, (n, k))))
        n_out = n // 2 if act == 2 else n
        y_ref = torch.empty((m, n_out), dtype=torch.float16, device="cuda")
        _reference(lib, x, m, k, act, wq, ws, n, y_ref)
        y = torch.full((m, n_out), float("nan"), dtype=torch.float16, device="cuda")
        torch.cuda.synchronize()
        before = torch.cuda.memory_stats()["allocation.all.allocated"]
        st = lib.rq_fp8_linear_noalloc(_p(x), m, k, act, _p(wq), _p(ws), n, _p(y), _stream())
        torch.cuda.synchronize()
        assert torch.cuda.memory_stats()["allocation.all.allocated"] == before
        assert st == 0, st
        assert np.array_equal(host(y).view(np.uint16), host(y_ref).view(np.uint16))


def test_noalloc_rejects_more_than_its_buffer():
    require_gpu()
    from fp8_quantized_generative_amd import _lib
    lib = _lib.load()
    case("noalloc: sizes beyond the static buffer")
    k = 8192
    m = _lib.RQ_STATIC_SCRATCH_BYTES // k  # its rows alone fill the buffer; the scales do not fit
    x = torch.zeros((1, k), dtype=torch.float16, device="cuda")  # never read: rejected first
    wq = torch.zeros((16, k), dtype=torch.uint8, device="cuda")
    ws = torch.ones(16, dtype=torch.float32, device="cuda")
    y = torch.zeros((1, 16), dtype=torch.float16, device="cuda")
    assert lib.rq_fp8_linear_noalloc(_p(x), m, k, 0, _p(wq), _p(ws), 16, _p(y), _stream()) == _lib.RQ_ERR_SCRATCH
    # the largest accepted size at this K runs
    m_ok = m
    while lib.rq_fp8_linear_workspace_size(m_ok, k, 0) > _lib.RQ_STATIC_SCRATCH_BYTES:
        m_ok -= 1
    assert lib.rq_fp8_linear_noalloc(_p(x), m_ok + 1, k, 0, _p(wq), _p(ws), 16, _p(y), _stream()) == \
        _lib.RQ_ERR_SCRATCH
    x2 = torch.zeros((m_ok, k), dtype=torch.float16, device="cuda")
    y2 = torch.full((m_ok, 16), 1.0, dtype=torch.float16, device="cuda")
    assert lib.rq_fp8_linear_noalloc(_p(x2), m_ok, k, 0, _p(wq), _p(ws), 16, _p(y2), _stream()) == 0
    torch.cuda.synchronize()
    assert not torch.any(y2).item()
