"""Host-side pieces of bench.py (no GPU): the roofline record and the --gpus guard."""
import subprocess
import sys

import pytest

import bench


def test_roofline_mfma_bound_at_the_headline_shape():
    M = N = K = 8192
    flops, nbytes = 2.0 * M * N * K, 2 * (M * K + K * N + M * N)
    rec = bench.roofline(flops, nbytes, 0.85, bench.PEAK_TFLOPS_F16, None)
    assert rec["bound"] == "mfma" and rec["unit"] == "TFLOP/s"
    assert rec["achieved"] == pytest.approx(flops / 0.85e-3 / 1e12, rel=1e-4)
    assert rec["frac"] == pytest.approx(rec["achieved"] / bench.PEAK_TFLOPS_F16, abs=1e-4)
    assert rec["intensity"] > rec["ridge"]


def test_roofline_hbm_bound_for_a_skinny_shape():
    M, N, K = 64, 8192, 8192
    flops, nbytes = 2.0 * M * N * K, 2 * (M * K + K * N + M * N)
    rec = bench.roofline(flops, nbytes, 0.0289, bench.PEAK_TFLOPS_F16, None)
    assert rec["bound"] == "hbm" and rec["unit"] == "GB/s" and rec["peak"] == 8000.0
    assert rec["achieved"] == pytest.approx(nbytes / 0.0289e-3 / 1e9, rel=1e-3)
    assert rec["frac"] == pytest.approx(rec["achieved"] / 8000.0, abs=1e-4)
    # the ridge of the fp16 peak against 8 TB/s
    assert rec["ridge"] == pytest.approx(bench.PEAK_TFLOPS_F16 * 1e12 / 8e12, abs=0.1)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], capture_output=True, text=True,
                       cwd=bench.ROOT, timeout=300)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr) or "1 GPU" in (r.stdout + r.stderr)


def test_cpu_table_times_the_oracle_over_a_whole_workload(capsys):
    import json
    import bench
    bench.cpu_table(["gemm_relu_f16_256"])
    recs = [json.loads(line) for line in capsys.readouterr().out.splitlines() if line.startswith("{")]
    # one run on all host threads, one on a single thread for the smallest square workload
    assert [r["workload"] for r in recs] == ["gemm_relu_f16_256"] * 2
    assert recs[1]["threads"] == 1
    for r in recs:
        assert r["oracle_s"] > 0
        assert abs(r["oracle_gflops"] - 2 * 256 ** 3 / r["oracle_s"] / 1e9) <= 0.01 * r["oracle_gflops"] + 0.01
