"""Host-side logic of bench.py: the step's dispatch table, matching a profile's kernel
sequence to calls, the traffic scaling, and the one-GPU contract.  No GPU needed."""

import json
import subprocess
import sys

import pytest

import bench


def _names(only=None, steps=2, prefix=("quant_rows_regs<4, false>", "at::native::fill")):
    tok = {"quant": "void rq::quant_rows_regs<8, false>(...)", "gemm": "void rq::gemm_fp8_kernel<Cfg>(...)",
           "reduce": "void rq::splitk_reduce<false>(...)", "plan": "void rq::plan_single<1>(...)",
           "plan_hist": "rq::plan_hist(...)", "plan_scan": "rq::plan_scan(...)", "plan_scatter": "rq::plan_scatter(...)",
           "combine": "rq::combine_kernel(...)"}
    seq = [tok[k] for _, k in bench.step_dispatches(only)]
    return list(prefix) + seq * steps + ["at::native::vectorized_elementwise_kernel (copy)"]


def test_step_table_matches_workloads():
    seq = bench.step_dispatches(None)
    # 8 linears x 2 kernels plus the split-K reduce of the small-M down projection; the 32768-slot
    # gate/up MoE call x 5 (three plan kernels, quantizer, GEMM), the 1024-slot one x 3 (one plan
    # kernel); 2 down calls x 3 (they reuse the plan: quantizer, GEMM, combine)
    assert len(seq) == 8 * 2 + 1 + 5 + 3 + 2 * 3
    assert ("moe gate_up", "gemm") in seq and ("moe down", "plan") not in seq
    assert ("layer_small_m down", "reduce") in seq and ("moe gate_up", "plan_scan") in seq
    assert len(bench.step_dispatches("moe")) == 8


def test_align_finds_every_step_and_labels():
    names = _names(steps=3)
    aligned, n = bench._align_steps(names, None, None)
    assert n == 3
    labels = [(label, kind) for _, label, kind in aligned]
    assert labels == bench.step_dispatches(None) * 3
    # the weight-quantization dispatch before the steps is not picked
    assert min(i for i, _, _ in aligned) == 2


def test_align_rejects_a_foreign_sequence():
    names = ["rq::plan_single(...)"] * 5
    with pytest.raises(SystemExit):
        bench._align_steps(names, None, None)


def test_traffic_scaling(tmp_path):
    res = {"fetch_size_kib_per_launch": 1000.0, "write_size_kib_per_launch": 300.0,
           "copy_fetch_size_kib": 256.0 * 1024, "copy_write_size_kib": 512.0 * 1024}
    out = tmp_path / "t.json"
    bench.finish_traffic(res, 512, str(out), 10 ** 6)
    t = json.loads(out.read_text())
    assert t["fetch_factor"] == 0.5 and t["write_factor"] == 1.0
    assert t["traffic_bytes_per_launch"] == int(1000 * 1024 / 0.5 + 300 * 1024)
    assert t["algorithmic_bytes_per_launch"] == 10 ** 6


def test_algorithmic_bytes_of_the_dominant_call():
    r, k, n, e = 32768, 2048, 8192, 32
    assert bench.dominant_algorithmic_bytes() == r * k + e * n * k + 4 * (r + e * n) + 2 * r * (n // 2)


def test_algorithmic_bytes_of_the_largest_quantizer_call():
    r, k = 32768, 4096
    assert bench.quant_algorithmic_bytes() == 2 * r * k + r * k + 4 * r


def test_more_than_one_gpu_exits_with_a_message():
    p = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"], capture_output=True, text=True)
    assert p.returncode == 2 and "one GPU" in p.stderr


def test_stats_us_percentiles():
    st = bench.stats_us([i / 1000.0 for i in range(1, 101)])  # 1..100 us given in ms
    assert st["n"] == 100 and st["median"] == 50.5 and st["mean"] == 50.5
    assert st["p10"] == pytest.approx(10.9) and st["p90"] == pytest.approx(90.1)


def test_stored_trace_needs_matching_sources(tmp_path):
    good = tmp_path / "t.txt"
    sha = bench.source_hash(bench.GEMM_SOURCES)
    good.write_text("# x\n# dominant launch (moe gate_up grouped GEMM) sources sha256_16: %s\n"
                    "# dominant launch (moe gate_up grouped GEMM): avg 512.25 us over 25 calls\n" % sha)
    assert bench.stored_trace_us(str(good)) == 512.25
    stale = tmp_path / "s.txt"
    stale.write_text(good.read_text().replace(sha, "0" * 16))
    assert bench.stored_trace_us(str(stale)) is None
    assert bench.stored_trace_us(str(tmp_path / "missing.txt")) is None
