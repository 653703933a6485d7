"""bench.py's host logic that needs no GPU: the committed counter summaries
parse, name the three kernels, and are attached only to the workload (and
kernel sources) they were taken on."""

import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
STAGES = ("pass1", "pass2_query", "pass2_key")


def test_committed_counter_files_parse():
    t = json.load(open(bench.TRAFFIC_FILE))
    m = json.load(open(bench.MFMA_FILE))
    for f in (t, m):
        assert len(f["kernel_source_sha256_16"]) == 16
        assert f["workload"] == "bob_b1h4n65536d64_bf16"
    assert set(t["bytes_per_launch"]) == set(STAGES)
    assert set(t["bytes_per_launch_causal"]) == set(STAGES)
    for st in STAGES:
        k = m["kernels"][st]
        assert 0 < k["mfma_util"] < 1 and 1.0 < k["sclk_ghz"] < 2.5
        # the MFMA instructions counted are the products the launch is known
        # to execute (pass 2 recomputes the score tiles in both sweeps)
        assert abs(k["executed_products"] - k["executed_units_nominal"]) < 1e-6
        assert k["executed_units_nominal"] == bench.executed_units(False)[st]


def test_counters_only_for_their_workload():
    for st in STAGES:
        assert bench.measured_traffic(st, False, "bob_b1h8n16384d128_bf16") is None
        assert bench.measured_mfma(st, "bob_b1h1n262144d64_bf16") is None


def test_counters_only_for_their_kernel_sources(monkeypatch):
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0" * 16)
    for st in STAGES:
        assert bench.measured_traffic(st) is None
        assert bench.measured_mfma(st) is None


def test_multi_gpu_request_exits_with_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_step_accounting_credits_the_method_not_the_launches():
    """Pass 2 is credited as one step with the method's 12 products over the
    sum of its two launches' times (the launches execute 9 + 8), pass 1 with
    5; the whole call's 17 match the 34 B H N^2 d flop convention."""
    unit = 2.0 * 1 * 4 * 65536 ** 2 * 64
    ms = {"pass1": 10.0, "pass2_query": 16.0, "pass2_key": 15.0}
    acc = bench.step_accounting(ms, unit, 2500.0)
    assert acc["pass1"]["units"] == 5 and acc["pass2"]["units"] == 12
    assert acc["pass2"]["ms"] == 31.0 and acc["pass2"]["launches"] == ["pass2_query", "pass2_key"]
    assert abs(acc["pass2"]["tflops"] - 12 * unit / 31e-3 / 1e12) < 0.01
    assert sum(bench.method_units(False).values()) * unit == 34.0 * 4 * 65536 ** 2 * 64
    assert sum(bench.executed_units(False).values()) == 22
    fb = bench.step_accounting(ms, unit, 2500.0, first_backward=True)
    assert fb["pass2"]["units"] == 15 and sum(bench.executed_units(True).values()) == 25
