"""Host-side logic of bench.py (no GPU): the algorithmic bytes each bench line
divides by, the refusal of more than one GPU, and the traffic figures being
reported only for the kernel source they were measured on."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synthetic  # noqa: E402


@pytest.fixture(scope="module")
def ngq():
    import groupwise_int_weight_amd as g

    g.lib()  # host-only size queries below; no HIP call
    return g


@pytest.mark.parametrize("name,T,n_out,expect", [
    # packed weights + scales + X + Y, each once
    ("qk", 8, None, 5120 * 8192 // 2 + 80 * 8192 * 2 + 2 * 8 * 5120 + 2 * 8 * 8192),
    ("qk", 1, None, 5120 * 8192 // 2 + 80 * 8192 * 2 + 2 * 5120 + 2 * 8192),
    ("gv", 8, None, 5120 * 12288 * 5 // 8 + 80 * 12288 * 2 + 2 * 8 * 5120 + 2 * 8 * 12288),
    ("gate_up", 8, synthetic.N_FF, 5120 * 34816 // 2 + 80 * 34816 * 2 + 2 * 8 * 5120 + 2 * 8 * 17408),
    ("down", 8, None, 17408 * 5120 // 2 + 272 * 5120 * 2 + 2 * 8 * 17408 + 2 * 8 * 5120),
])
def test_algorithmic_bytes(ngq, name, T, n_out, expect):
    assert bench.algorithmic_bytes(ngq, synthetic.WORKLOADS[name], T, n_out=n_out) == expect


def test_headline_bytes_match_the_quoted_figures(ngq):
    # the per-launch figures the roofline and the profiles divide by
    assert bench.algorithmic_bytes(ngq, synthetic.WORKLOADS["qk"], 8) == 22495232
    assert bench.algorithmic_bytes(ngq, synthetic.WORKLOADS["gv"], 8) == 41566208


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_traffic_only_for_the_measured_source(tmp_path, monkeypatch):
    d = {"kernel_sha": bench.kernel_sha(), "workloads": {"qk_T8": {"bytes_per_launch": 123.0}}}
    f = tmp_path / "traffic.json"
    f.write_text(json.dumps(d))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.traffic_for("qk", 8) == 123.0
    assert bench.traffic_for("gv", 8) is None
    d["kernel_sha"] = "0" * 16
    f.write_text(json.dumps(d))
    assert bench.traffic_for("qk", 8) is None


def test_kernel_hash_ignores_comments_only(tmp_path, monkeypatch):
    code = "int f(int a) {\n  return a + 1;  // one more\n}\n"
    src = tmp_path / "k.hip"
    src.write_text(code)
    monkeypatch.setattr(bench, "KERNEL_SRC", str(src))
    h = bench.kernel_sha()
    src.write_text("/* a block\n   comment */\n" + code.replace("// one more", "// a different note") + "\n\n")
    assert bench.kernel_sha() == h
    src.write_text(code.replace("a + 1", "a + 2"))
    assert bench.kernel_sha() != h


def test_summarize_trace_percentiles(tmp_path):
    """bench.py --summarize-trace: per-kernel median, p10 and p90 of a
    rocprofv3 kernel-trace CSV (durations from the timestamps, in us)."""
    import bench

    p = tmp_path / "kernel_trace.csv"
    rows = ["Kernel_Name,Start_Timestamp,End_Timestamp"]
    for i in range(11):  # durations 1..11 us
        rows.append(f"gemm_a,{1000 * i},{1000 * i + 1000 * (i + 1)}")
    rows.append("other,0,500")
    p.write_text("\n".join(rows) + "\n")
    out = {r["kernel"]: r for r in bench.summarize_trace(str(p))}
    a = out["gemm_a"]
    assert a["calls"] == 11 and a["median_us"] == 6.0 and a["p10_us"] == 2.0 and a["p90_us"] == 10.0
    assert out["other"]["calls"] == 1 and out["other"]["median_us"] == 0.5
