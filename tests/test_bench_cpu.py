"""The measurement harness on the CPU: bench.py's refusal of more than one
GPU, its per-call arithmetic, the counter-based traffic it reports only for
the kernel sources the counters were taken on, and the command lines the
GPU-free parent gives its child processes. Nothing here touches a GPU."""
import json
import os
import subprocess
import sys
import types

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
    assert res.stdout == ""


def test_per_call_fraction_and_budget():
    # 2.4 GB in 0.4 ms is 6 TB/s, 0.75 of 8 TB/s; 70% of peak allows 0.4286 ms
    pc = bench.per_call(2_400_000_000, 0.4)
    assert pc["step_GBps"] == pytest.approx(6000.0)
    assert pc["step_frac"] == pytest.approx(0.75)
    assert pc["budget_ms_at_70pct"] == pytest.approx(2.4e9 / (0.7 * 8e12) * 1e3)


@pytest.mark.parametrize("workload", bench.WORKLOADS)
def test_counter_traffic_only_for_the_sources_it_was_taken_on(workload, monkeypatch):
    kv = bench.counter_summary(workload)
    assert kv.get("workload") == workload
    assert int(kv["hbm_bytes_per_launch"]) > 0
    monkeypatch.setattr(bench, "kernel_source_digest", lambda: kv["kernel_source_sha256_16"])
    assert bench.read_counter_traffic(workload) == int(kv["hbm_bytes_per_launch"])
    monkeypatch.setattr(bench, "kernel_source_digest", lambda: "0" * 16)
    assert bench.read_counter_traffic(workload) is None


def test_parent_runs_every_workload_in_a_child(monkeypatch, capsys):
    """The parent starts one child per workload: the headline with the steps
    asked for and the extra entry points, the others on at least SMALL_STEPS
    steps, each with about five event pairs; it prints one JSON line."""
    calls = []

    def fake_run(cmd, stdout=None, text=None, timeout=None):
        calls.append(cmd)
        name = cmd[cmd.index("--workload") + 1]
        steps = int(cmd[cmd.index("--steps") + 1])
        res = {"metric": "m", "value": 1.0, "steps": steps, "ms_per_step": 0.5,
               "config": {"workload": name, "valid_positions_per_s": 1.0,
                          "algorithmic_bytes": 10,
                          "per_call": bench.per_call(10, 0.5),
                          "draw_reread": {"bytes": 0}},
               "roofline": {"kernel_us_mean": 1.0, "frac": 0.5, "traffic": None}}
        return types.SimpleNamespace(returncode=0, stdout=json.dumps(res) + "\n")

    monkeypatch.setattr(bench.subprocess, "run", fake_run)
    monkeypatch.setattr(sys, "argv", ["bench.py", "--steps", "20", "--event-every", "4"])
    args = bench.parse_args()
    assert bench.parent(args) == 0
    names = [c[c.index("--workload") + 1] for c in calls]
    assert names == list(bench.WORKLOADS)
    for c in calls:
        name = c[c.index("--workload") + 1]
        steps = int(c[c.index("--steps") + 1])
        every = int(c[c.index("--event-every") + 1])
        if name == bench.HEADLINE:
            assert (steps, every) == (20, 4) and "--extras" in c
        else:
            assert steps >= bench.SMALL_STEPS and "--extras" not in c
            assert steps // every == 5
    line = json.loads(capsys.readouterr().out.strip().splitlines()[-1])
    assert set(line["configs"]) == set(bench.WORKLOADS)
    assert line["steps"] == 20
    # with the default steps the headline too samples about five steps
    monkeypatch.setattr(sys, "argv", ["bench.py"])
    calls.clear()
    assert bench.parent(bench.parse_args()) == 0
    head = next(c for c in calls if c[c.index("--workload") + 1] == bench.HEADLINE)
    steps = int(head[head.index("--steps") + 1])
    every = int(head[head.index("--event-every") + 1])
    assert steps == bench.SMALL_STEPS and steps // every == 5
