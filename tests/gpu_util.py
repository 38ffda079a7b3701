"""Helpers shared by the GPU parity tests (device transfer and case logging only)."""

import sys

import numpy as np
import pytest
import torch


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fp8_quantized_generative_amd as rq  # fails loudly if the library is missing
    from fp8_quantized_generative_amd import _lib
    assert _lib.load().rq_device_supported(torch.cuda.current_device()) == 1, "device is not gfx950"
    return rq


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def case(msg):
    """Name the case on stderr before a GPU step, flushed, so a crash still names it."""
    print("[case] " + msg, file=sys.stderr, flush=True)


def ulp_diff16(a, b):
    """|a - b| in FP16 units of the last place, via the ordered integer encoding."""
    ai = np.asarray(a, np.float16).view(np.int16).astype(np.int64)
    bi = np.asarray(b, np.float16).view(np.int16).astype(np.int64)
    ai = np.where(ai < 0, -(ai & 0x7FFF), ai)
    bi = np.where(bi < 0, -(bi & 0x7FFF), bi)
    return np.abs(ai - bi)
