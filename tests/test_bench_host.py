"""Host-side pieces of bench.py (no GPU): the CPU baselines on a small workload, the
traffic-summary lookup, the rocprofv3 summarisers, and the refusal of more than one GPU."""
import os
import subprocess
import sys

import bench
from quantized_attention_video_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_cpu_baseline_small_sample():
    w = W.get("fixed_q128_kv192")
    r = bench.cpu_baseline(w, W.make_inputs(w), att_heads=1, rows=64)
    assert r["kind"] == "oracle" and r["unit"] == "TOPS" and r["value"] > 0 and r["cores"] >= 1
    assert "extrapolated" in r["sample"]


def test_cpu_baseline_packed_and_batched():
    """The sampled baseline extrapolates by operation count, so it also covers packed
    segments and batches of several sequences."""
    tiny = W.Workload("tiny_packed", 99, H=2, seqlens=[100, 37, 0, 5], layout="packed")
    r = bench.cpu_baseline(tiny, W.make_inputs(tiny), att_heads=1, rows=16)
    assert r["value"] > 0 and "segment" in r["sample"]
    w = W.get("ragged_b2_h16_l1000")
    small = W.Workload("tiny_batch", 98, H=2, B=2, Lq=70, Lk=90, layout="blhd")
    r = bench.cpu_baseline(small, W.make_inputs(small), att_heads=1, rows=16)
    assert r["value"] > 0 and "sequence" in r["sample"]
    assert w.ops() == 4 * 2 * 1000 * 1000 * 128 * 16


def test_cpu_oracle_full_small_shape():
    w = W.get("fixed_q128_kv192")
    r = bench.cpu_oracle_full(w, W.make_inputs(w))
    assert r["kind"] == "oracle" and r["unit"] == "us" and r["value"] > 0 and r["single_thread_us"] > 0
    assert r["cores"] >= 1


def test_traffic_summary_lookup(tmp_path, monkeypatch):
    f = tmp_path / "traffic.txt"
    f.write_text("# comment\nworkload = h3_video_l37810\n"
                 f"attn_hip_sha256_16 = {bench.kernel_source_hash()}\nhbm_bytes_per_launch = 123456\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic("h3_video_l37810") == 123456.0
    assert bench.measured_traffic("dense_h8_l4096") is None  # another workload
    f.write_text("workload = h3_video_l37810\nattn_hip_sha256_16 = 0000\nhbm_bytes_per_launch = 1\n")
    assert bench.measured_traffic("h3_video_l37810") is None  # taken from another kernel source


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert p.returncode == 2 and "one GPU" in p.stderr


def test_percentiles_and_cv():
    xs = [4.0, 1.0, 3.0, 2.0, 5.0]
    assert bench._pct(xs, 0) == 1.0 and bench._pct(xs, 50) == 3.0 and bench._pct(xs, 100) == 5.0
    assert bench._pct(xs, 10) == 1.4
    assert abs(bench._cv([2.0, 4.0]) - 1.0 / 3.0) < 1e-12


def test_trace_and_counter_summaries(tmp_path, capsys):
    """The rocprofv3 summarisers: warm-up and timed launches apart when a kernel ran
    steps + warmup times; per-dispatch sums of a counter's dimensions, averaged over the
    timed dispatches."""
    import csv

    trace = tmp_path / "t_kernel_trace.csv"
    with open(trace, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        t = 0
        for i in range(5):  # 2 warm-up + 3 timed launches of one step kernel: 10, 20, 30, 40, 50 us
            w.writerow(["void sattn::attn_fwd_kernel<false, true>(sattn::AttnParams)", t, t + 10000 * (i + 1)])
            t += 100000
        w.writerow(["__amd_rocclr_copyBuffer", t, t + 7000])
    bench.summarize_trace(str(trace), steps=3, warmup=2)
    out = capsys.readouterr().out.splitlines()
    timed = [ln.split() for ln in out if " timed " in ln]
    warm = [ln.split() for ln in out if " warm-up " in ln]
    assert len(timed) == 1 and timed[0][-5] == "3" and float(timed[0][-4]) == 40.0  # mean of 30, 40, 50
    assert len(warm) == 1 and warm[0][-5] == "2" and float(warm[0][-4]) == 15.0
    assert any("copyBuffer" in ln and " all " in ln and "7.0" in ln for ln in out)

    cnt = tmp_path / "c_counter_collection.csv"
    with open(cnt, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Counter_Name", "Dispatch_Id", "Counter_Value"])
        for d in range(3):  # 1 warm-up + 2 timed dispatches, each counter reported in two dimensions
            for part in (1.0, 2.0):
                w.writerow(["stats_q_kernel(int)", "FETCH_SIZE", d + 1, part * (d + 1)])
    bench.summarize_counters([str(cnt)], steps=2, warmup=1)
    line = capsys.readouterr().out.strip()
    assert "stats_q_kernel" in line and "FETCH_SIZE" in line and "n=  2" in line
    assert line.endswith("mean=7.5")  # (3*2 + 3*3) / 2: the two timed dispatches, dimensions summed
