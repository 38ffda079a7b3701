"""Pins of the oracle's SiLU*up intermediate and MoE plan / grouped linear / combine.

MoE: page "Quantized Inference for OneRec-V2：生成式推荐开始直接吃 LLM 量化栈", section
关键证据 (the MoE grouped GEMM is quantized) and page "FP8量化在生成式推荐系统OneRec-V2
中的优化实践", §2.1 (the routing gate stays FP16, so ids and weights are inputs).
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import ffn, linear, moe, quant
import workloads


def test_silu_mul_matches_torch_silu():
    rng = np.random.default_rng(1)
    gu = (rng.standard_normal((64, 2 * 96)) * 4).astype(np.float16)
    gu[0, :4] = np.float16([0.0, -0.0, 30000.0, -30000.0])
    h = ffn.silu_mul(gu, 96)
    g = torch.from_numpy(gu[:, :96].astype(np.float64))
    u = torch.from_numpy(gu[:, 96:].astype(np.float64))
    with np.errstate(over="ignore"):
        ref = (torch.nn.functional.silu(g) * u).numpy().astype(np.float16)
    assert np.array_equal(h.view(np.uint16) & 0x7FFF, ref.view(np.uint16) & 0x7FFF)


def test_silu_mul_closed_forms_and_operand_order():
    gu = np.array([[0.0, 20.0, -30.0, 1.0, 3.0, 2.0, 2.0, 5.0]], np.float16)
    h = ffn.silu_mul(gu, 4)
    # silu(0) = 0; silu(20) = 20 to FP16 precision; silu(-30) * 2 ~ -5.6e-12 rounds to -0;
    # silu(1) * 5 = 5 / (1 + e^-1)
    assert h[0, 0] == 0 and h[0, 1] == np.float16(20.0 * 2.0)
    assert h[0, 2] == 0 and np.signbit(h[0, 2])
    assert h[0, 3] == np.float16(5.0 / (1.0 + np.exp(-1.0)))
    swapped = ffn.silu_mul(np.concatenate([gu[:, 4:], gu[:, :4]], axis=1), 4)
    assert not np.array_equal(swapped, h)


def _brute_plan(ids, e_count):
    t, k = ids.shape
    pairs = sorted((int(ids[tt, kk]), tt * k + kk) for tt in range(t) for kk in range(k))
    perm = [j for _, j in pairs]
    counts = [sum(1 for e, _ in pairs if e == x) for x in range(e_count)]
    offsets = [0]
    for c in counts:
        offsets.append(offsets[-1] + c)
    return counts, offsets, perm


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_plan_matches_sorted_pairs(seed):
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, 7, size=(23, 3))
    counts, offsets, perm, pos = moe.plan(ids, 9)   # experts 7 and 8 empty
    c, o, p = _brute_plan(ids, 9)
    assert counts.tolist() == c and offsets.tolist() == o and perm.tolist() == p
    assert np.array_equal(perm[pos], np.arange(ids.size))


def _expert_weights(rng, e, n, k):
    w = (rng.standard_normal((e, n, k)) * 0.05).astype(np.float16)
    wq = np.empty((e, n, k), np.uint8)
    sw = np.empty((e, n), np.float32)
    for i in range(e):
        wq[i], sw[i] = quant.quantize_rows(w[i])
    return w, wq, sw


def test_all_tokens_on_one_expert_equals_dense_linear():
    rng = np.random.default_rng(3)
    t, k, n, e = 17, 64, 32, 4
    x = rng.standard_normal((t, k)).astype(np.float16)
    _, wq, sw = _expert_weights(rng, e, n, k)
    ids = np.full((t, 1), 2)
    out = moe.grouped_linear(x, moe.IN_TOKENS, moe.ACT_NONE, ids, wq, sw)
    dense = linear.linear(*quant.quantize_rows(x), wq[2], sw[2])
    assert np.array_equal(out["y"], dense)


def test_top1_unit_weight_combine_is_identity():
    rng = np.random.default_rng(4)
    t, k, n, e = 19, 32, 16, 5
    x = rng.standard_normal((t, k)).astype(np.float16)
    _, wq, sw = _expert_weights(rng, e, n, k)
    ids = rng.integers(0, e, size=(t, 1))
    w1 = np.ones((t, 1), np.float16)
    out = moe.grouped_linear(x, moe.IN_TOKENS, moe.ACT_NONE, ids, wq, sw, moe.OUT_COMBINED, w1)
    for tt in range(t):
        assert np.array_equal(out["y"][tt], out["y_perm"][out["pos"][tt]])
        row = linear.linear(*quant.quantize_rows(x[tt:tt + 1]), wq[ids[tt, 0]], sw[ids[tt, 0]])
        assert np.array_equal(out["y"][tt], row[0])


def test_token_order_invariance_and_quantize_before_dispatch():
    rng = np.random.default_rng(5)
    t, k, n, e, top_k = 21, 48, 16, 6, 2
    x = rng.standard_normal((t, k)).astype(np.float16)
    _, wq, sw = _expert_weights(rng, e, n, k)
    ids = np.stack([rng.permutation(e)[:top_k] for _ in range(t)])
    w = rng.random((t, top_k)).astype(np.float16)
    base = moe.grouped_linear(x, moe.IN_TOKENS, moe.ACT_NONE, ids, wq, sw, moe.OUT_COMBINED, w)
    p = rng.permutation(t)
    shuf = moe.grouped_linear(x[p], moe.IN_TOKENS, moe.ACT_NONE, ids[p], wq, sw, moe.OUT_COMBINED, w[p])
    assert np.array_equal(shuf["y"], base["y"][p])
    # PERMUTED input: the gathered FP16 rows, quantized after dispatch
    gathered = x[base["perm"] // top_k]
    after = moe.grouped_linear(gathered, moe.IN_PERMUTED, moe.ACT_NONE, ids, wq, sw)
    assert np.array_equal(after["y"], base["y_perm"])


def test_combine_matches_fraction_brute_force():
    rng = np.random.default_rng(6)
    t, top_k, n, r = 5, 3, 4, 15
    y = rng.standard_normal((r, n)).astype(np.float16)
    w = rng.random((t, top_k)).astype(np.float16)
    pos = rng.permutation(r)
    out = moe.combine(y, pos, w)
    for tt in range(t):
        for j in range(n):
            s = sum(Fraction(float(w[tt, kk])) * Fraction(float(y[pos[tt * top_k + kk], j]))
                    for kk in range(top_k))
            assert out[tt, j] == np.float16(float(s))


def test_empty_expert_reads_no_weights():
    rng = np.random.default_rng(7)
    t, k, n, e = 12, 32, 16, 4
    x = rng.standard_normal((t, k)).astype(np.float16)
    _, wq, sw = _expert_weights(rng, e, n, k)
    ids = rng.integers(0, 3, size=(t, 2))       # expert 3 never routed
    a = moe.grouped_linear(x, moe.IN_TOKENS, moe.ACT_NONE, ids, wq, sw)
    wq2 = wq.copy()
    wq2[3] = 0x7F                               # NaN bytes: would poison any read
    b = moe.grouped_linear(x, moe.IN_TOKENS, moe.ACT_NONE, ids, wq2, sw)
    assert np.array_equal(a["y"], b["y"])


def test_silu_permuted_call_chain():
    rng = np.random.default_rng(9)
    t, k, f, e = 10, 32, 16, 3
    ids = np.stack([rng.permutation(e)[:2] for _ in range(t)])
    gu = rng.standard_normal((t * 2, 2 * f)).astype(np.float16)
    _, wq, sw = _expert_weights(rng, e, k, f)
    out = moe.grouped_linear(gu, moe.IN_PERMUTED, moe.ACT_SILU_MUL, ids, wq, sw)
    h = ffn.silu_mul(gu, f)
    assert np.array_equal(out["h"], h)
    hq, hs = quant.quantize_rows(h)
    for ee in range(e):
        lo, hi = out["offsets"][ee], out["offsets"][ee + 1]
        ref = linear.linear(hq[lo:hi], hs[lo:hi], wq[ee], sw[ee])
        assert np.array_equal(out["y"][lo:hi], ref)


def test_zipf_routing_recipe():
    data = workloads.make(4, t=4096, k=64, f=32)
    ids = data["ids"]
    counts = np.bincount(ids.reshape(-1), minlength=32)
    assert (counts == 0).sum() >= 1
    assert np.all(ids[:, 0] != ids[:, 1])
    assert counts.max() > 4 * np.median(counts[counts > 0])
    assert np.allclose(data["topk_w"].astype(np.float64).sum(axis=1), 1.0, atol=2e-3)


def test_gate_up_order_is_a_block_permutation():
    o = ffn.gate_up_order(96)
    assert sorted(o.tolist()) == list(range(192))
    # blocks of 32: gate features 0..31, up features 0..31, gate 32..63, ...
    assert o[:32].tolist() == list(range(32)) and o[32:64].tolist() == list(range(96, 128))
    assert o[64:96].tolist() == list(range(32, 64)) and o[-32:].tolist() == list(range(160, 192))
    with pytest.raises(ValueError):
        ffn.gate_up_order(48)


def test_gate_silu_of_reordered_weights_equals_silu_mul():
    # reordering W_gu's rows reorders the linear's output columns, so the gated output of the
    # reordered weights is silu_mul of the plain layout, bit for bit
    rng = np.random.default_rng(11)
    f, k = 64, 48
    x = workloads.acts_outliers(rng, 9, k)
    w = workloads.weights(rng, (2 * f, k))
    xq, xs = quant.quantize_rows(x)
    wq, ws = quant.quantize_rows(w)
    plain = linear.linear(xq, xs, wq, ws)
    o = ffn.gate_up_order(f)
    gated = linear.linear(xq, xs, wq[o], ws[o])
    assert np.array_equal(gated.view(np.uint16), plain[:, o].view(np.uint16))
    h = ffn.gate_silu(gated)
    assert np.array_equal(h.view(np.uint16), ffn.silu_mul(plain, f).view(np.uint16))
    # a plain-layout output fed to gate_silu is a different function (the layouts are not mixed up)
    assert not np.array_equal(ffn.gate_silu(plain).view(np.uint16), h.view(np.uint16))
