"""CPU checks of the benchmark's contract (no GPU needed).

bench.py takes the HBM traffic and VALU instruction counts of the attention
kernel from committed rocprofv3 summaries under profiles/, and only while the
kernel-source hash stored there matches the current sources.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_committed_profiles_match_the_kernel_sources():
    # a kernel change must be followed by new counter summaries
    traffic = bench.measured_traffic()
    assert traffic is not None
    assert 0.9 * 301989888 < traffic < 3 * 301989888   # algorithmic bytes 6N at S=16384, H=24
    v = bench.valu_issue(1.6)
    assert v is not None
    assert 0.0 < v["frac"] < 1.0
    assert v["slots_per_launch"] > 0


def test_profile_from_another_kernel_source_is_ignored(tmp_path):
    p = tmp_path / "prof.txt"
    p.write_text("# comment = ignored\nhbm_bytes_per_launch = 123   # bytes\nkernel_hash = 0000000000000000\n")
    assert bench.profile_values(str(p), ["hbm_bytes_per_launch"]) is None
    p.write_text("hbm_bytes_per_launch = 123   # bytes\nkernel_hash = %s   # current\n" % bench.kernel_hash())
    assert bench.profile_values(str(p), ["hbm_bytes_per_launch"]) == [123.0]
    assert bench.profile_values(str(p), ["missing_key"]) is None


@pytest.mark.parametrize("name", ["attn_fwd_image_dit_2048_kernel_trace.txt", "attn_fwd_image_dit_2048_traffic.txt",
                                  "attn_fwd_image_dit_2048_valu.txt", "attn_fwd_all_workloads_bench.txt"])
def test_profile_summaries_state_their_command(name):
    text = open(os.path.join(ROOT, "profiles", name)).read()
    assert "bench.py" in text
    if "bench" not in name:
        assert "rocprofv3" in text


@pytest.mark.gpu
def test_bench_prints_one_json_line_with_the_contract_keys():
    import json
    print("bench.py --steps 2 --warmup 1 --no-cpu-baseline", flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "2", "--warmup", "1",
                        "--no-cpu-baseline"], capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "valu_issue"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 2 and d["warmup"] == 1
    assert d["value"] > 0 and d["config"]["workload"]
    roof = d["roofline"]
    assert roof["bound"] == "mfma" and roof["peak"] == 5000.0
    assert 0 < roof["frac"] < 1
    # the counter-derived figures are reported only while the committed
    # profile was taken on the current kernel sources, and are null otherwise
    import bench
    current = bench.profile_values(bench.TRAFFIC_PROFILE, ["hbm_bytes_per_launch"]) is not None
    assert (roof["traffic"] is not None) == current
    if roof["traffic"] is not None:
        assert roof["traffic"] > 0
    vcur = bench.profile_values(bench.VALU_PROFILE, ["valu_insts_per_launch"]) is not None
    assert (d["valu_issue"] is not None) == vcur
    if d["valu_issue"] is not None:
        assert 0 < d["valu_issue"]["frac"] < 1
