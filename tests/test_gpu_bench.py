"""bench.py end to end on the GPU (needs an MI355X): the one-line JSON of the throughput
mode on a mid-size dense shape and on the packed batch, and of the latency mode on the
fixed shape.  Each runs bench.py as a child process, as a user would."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CONTRACT = ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
            "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline")


def _bench(*args, timeout=300):
    print(f"[bench] {' '.join(args)}", file=sys.stderr, flush=True)
    p = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                       timeout=timeout)
    assert p.returncode == 0, p.stderr[-3000:]
    lines = [ln for ln in p.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, p.stdout[-2000:]
    return json.loads(lines[0])


def test_throughput_line_dense():
    d = _bench("--workload", "dense_h8_l4096", "--steps", "3", "--warmup", "1", "--no-cpu-baseline")
    assert all(k in d for k in CONTRACT)
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1 and d["higher_is_better"] is True
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["vs_baseline"] is None
    assert d["config"]["workload"] == "dense_h8_l4096" and d["cpu_baseline"] is None
    r = d["roofline"]
    assert r["bound"] == "mfma" and r["peak"] == 5000.0 and 0 < r["frac"] < 1
    assert abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-12
    assert r["traffic"] is None  # the committed counter summary is for the H3-like layer only
    # value counts the whole step, achieved only the attention launch
    assert d["value"] <= r["achieved"]


def test_throughput_line_packed():
    d = _bench("--workload", "varlen_h24_4seg", "--steps", "2", "--warmup", "1", "--no-cpu-baseline")
    assert all(k in d for k in CONTRACT)
    assert d["config"]["seqlens"] == [37810, 8192, 1536, 100] and "sattn_fwd_fused" in d["config"]["step"]
    assert 0 < d["roofline"]["frac"] < 1


def test_throughput_line_two_pass():
    d = _bench("--workload", "varlen_h24_4seg", "--steps", "2", "--warmup", "1", "--no-cpu-baseline", "--two-pass")
    assert all(k in d for k in CONTRACT)
    assert d["config"]["step"] == "sattn_quantize_qkv + sattn_fwd_varlen" and d["roofline"]["traffic"] is None
    assert 0 < d["roofline"]["frac"] < 1


def test_latency_line_fixed_shape():
    d = _bench("--latency", "--workload", "fixed_q128_kv192", "--samples", "20", "--warmup", "5",
               "--no-cpu-baseline")
    assert d["unit"] == "us" and d["higher_is_better"] is False
    assert d["graph_replays_match_eager"] is True
    g = d["graph_replay_us"]
    assert g["samples"] == 20 and 0 < g["p10"] <= g["p50"] <= g["p90"] < 1000
    assert d["value"] == g["p50"] and d["vs_baseline"] > 0
    assert d["config"]["forward_workspace"] is True and d["config"]["key_split"] is False  # 3 epochs: too few
