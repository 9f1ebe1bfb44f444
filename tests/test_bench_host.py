"""Host logic of bench.py, without a GPU: more than one GPU is refused with a message; every
measurement runs in a child process with the run's options, and one that fails there (an
error, a crash, a time-out) comes back as an error entry, while the main process still prints
its one JSON line."""

import json
import os
import subprocess
import sys
import types

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stderr and p.stdout == ""


def _args(**kw):
    a = dict(workload="tiny", reserve=None, no_cpu_baseline=True, steps=3, warmup=2,
             kernel_reps=4, prefetch="fused", percentile=None, cap_div=None)
    a.update(kw)
    return types.SimpleNamespace(**a)


def test_run_section_outcomes(monkeypatch):
    seen = []

    def fake(rc, out="", exc=None):
        def run(cmd, **kw):
            seen.append(cmd)
            if exc:
                raise exc
            return subprocess.CompletedProcess(cmd, rc, stdout=out)
        return run

    monkeypatch.setattr(bench.subprocess, "run", fake(0, 'log line\n{"x": 1}\n'))
    assert bench.run_section("loop", _args(reserve=7)) == {"x": 1}
    cmd = seen[-1]
    opt = lambda o: cmd[cmd.index(o) + 1]
    assert opt("--section") == "loop" and opt("--workload") == "tiny" and opt("--reserve") == "7"
    assert opt("--steps") == "3" and opt("--warmup") == "2" and opt("--kernel-reps") == "4"
    assert opt("--prefetch") == "fused" and "--no-cpu-baseline" in cmd and "--percentile" not in cmd
    monkeypatch.setattr(bench.subprocess, "run", fake(-11))
    assert "status -11" in bench.run_section("prefill", _args())["error"]
    monkeypatch.setattr(bench.subprocess, "run", fake(0, "no json here\n"))
    assert "error" in bench.run_section("prefill", _args())
    monkeypatch.setattr(bench.subprocess, "run",
                        fake(0, exc=subprocess.TimeoutExpired(["x"], 900)))
    assert "timed out" in bench.run_section("prefetch_modes", _args())["error"]


def test_section_child_reports_its_failure_as_json():
    # no GPU here: the child's measurement fails, and it says so in one JSON object
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--section", "loop",
                        "--workload", "tiny", "--no-cpu-baseline"], capture_output=True, text=True,
                       timeout=600)
    lines = [ln for ln in p.stdout.splitlines() if ln.startswith("{")]
    assert p.returncode == 0 and len(lines) == 1
    assert "error" in json.loads(lines[0])


def test_main_prints_one_line_whatever_fails(monkeypatch, capsys):
    calls = []

    def fake(name, args, timeout_s=900):
        calls.append(name)
        if name == "headline":
            return {"metric": bench.METRIC, "value": 1.0e9, "unit": "indexed tokens/s"}
        return {"error": "section process exited with status -11"}
    monkeypatch.setattr(bench, "run_section", fake)
    monkeypatch.setattr(sys, "argv", ["bench.py", "--workload", "tiny"])
    bench.main()
    lines = [ln for ln in capsys.readouterr().out.splitlines() if ln.strip()]
    assert len(lines) == 1
    d = json.loads(lines[0])
    assert d["value"] == 1.0e9 and calls[0] == "headline"
    assert all("error" in d[n] for n in ("prefill", "prefill_offload", "loop", "prefetch_modes"))
    # a failed headline still gives the line, with no value and the reason
    monkeypatch.setattr(bench, "run_section", lambda name, args, timeout_s=900: {"error": "boom"})
    monkeypatch.setattr(sys, "argv", ["bench.py", "--no-prefill", "--no-loop", "--no-prefetch-modes"])
    bench.main()
    lines = [ln for ln in capsys.readouterr().out.splitlines() if ln.strip()]
    d = json.loads(lines[-1])
    assert len(lines) == 1 and d["value"] is None and d["error"] == "boom" and d["metric"] == bench.METRIC
