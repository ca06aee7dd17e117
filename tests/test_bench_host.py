"""bench.py's host logic on the CPU: the one-GPU refusal, the input seed, and
the rule that HBM traffic is reported only from counter summaries taken on
the current kernel sources."""
import argparse
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_before_any_device_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_input_seed_defaults_to_the_workload_and_follows_the_flag():
    class Case:
        seed_base = 4000

    assert bench.input_seed(argparse.Namespace(seed=None), Case) == 4000
    assert bench.input_seed(argparse.Namespace(seed=7), Case) == 7
    assert bench.input_seed(argparse.Namespace(seed=0), Case) == 0


def test_kernel_source_digest_is_stable_and_short():
    d = bench.kernel_source_digest()
    assert d == bench.kernel_source_digest()
    assert len(d) == 16 and int(d, 16) >= 0


def test_traffic_only_from_counters_of_the_current_kernel_sources(monkeypatch):
    name = "large_channel_n64_c512_14"
    with open(os.path.join(ROOT, "profiles", f"traffic_{name}.json")) as f:
        t = json.load(f)
    assert t["workload"] == name
    assert t["hbm_bytes_per_launch"] > t["algorithmic_bytes_per_launch"] > 0
    monkeypatch.setattr(bench, "kernel_source_digest", lambda: t["kernel_source_digest"])
    assert bench.traffic_from_profiles(name, t["algorithmic_bytes_per_launch"]) == t["hbm_bytes_per_launch"]
    monkeypatch.setattr(bench, "kernel_source_digest", lambda: "0" * 16)
    assert bench.traffic_from_profiles(name, t["algorithmic_bytes_per_launch"]) is None
    assert bench.traffic_from_profiles("no_such_workload", 1.0) is None
