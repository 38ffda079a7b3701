"""Small-M serving layer (workload 5) at full size against the oracle, every row.

512 rows (32 requests x 16 beam rows) of Student-t(3) activations through one layer's
linears, in the order and formulation the benchmark times them: merged QKV (N = 6144), O,
the dense FFN (gate/up 2 x 8192 with the SiLU*up written from the gate/up epilogue, then
the down projection over K = 8192) and the top-2-of-32 expert FFN (F = 4096, Zipf-loaded
experts of a few rows each, one empty), the quantized paths of page "Quantized Inference
for OneRec-V2：生成式推荐开始直接吃 LLM 量化栈", section 关键证据, at the batch-32
serving shape of page "FP8量化在生成式推荐系统OneRec-V2中的优化实践", §4.1.

Every stage is checked: weight and activation bytes and scales bit-exact, every output
row of every GEMM within the linear tolerance, h within 1 FP16 ulp, the gated forms bit for
bit equal to the unfused ones, the combine within 1 FP16 ulp of the oracle's combine.
"""

import numpy as np
import pytest

import workloads
from tests import parity
from tests.gpu_util import require_gpu

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


@pytest.fixture(scope="module")
def layer():
    return workloads.make(5)


def test_layer_qkv_and_o(layer):
    rq = require_gpu()
    _, r1 = parity.linear_all_rows(rq, layer["x_qkv"], layer["w_qkv"], "workload 5: QKV 512 x 6144 x 2048", "slabs")
    _, r2 = parity.linear_all_rows(rq, layer["x_o"], layer["w_o"], "workload 5: O 512 x 2048 x 2048", "slabs")
    assert r1 <= 1 and r2 <= 1


def test_layer_dense_ffn(layer):
    rq = require_gpu()
    r_gu, r_dn = parity.dense_ffn_gated(rq, layer["x_ffn"], layer["w_gu"], layer["w_dn"],
                                        "workload 5: FFN 512 rows, F = 8192", "slabs")
    assert r_gu <= 1 and r_dn <= 1


def test_layer_expert_ffn(layer):
    rq = require_gpu()
    counts, r_gu, r_dn = parity.moe_ffn_gated(rq, layer["x_moe"], layer["ids"], layer["topk_w"],
                                              layer["w_gu_moe"], layer["w_dn_moe"],
                                              "workload 5: MoE 512 tokens, top-2 of 32, F = 4096", "slabs")
    assert (counts == 0).any() and counts.max() < 512
    assert r_gu <= 1 and r_dn <= 1
