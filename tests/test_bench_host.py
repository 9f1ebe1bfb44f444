"""Host logic of bench.py, without a GPU: more than one GPU is refused with a message, and a
secondary measurement that fails in its child process (an error, a crash, a time-out) comes
back as an error entry instead of taking the headline line with it."""

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
    a = dict(workload="tiny", reserve=None, no_cpu_baseline=True)
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
    assert cmd[cmd.index("--section") + 1] == "loop" and cmd[cmd.index("--workload") + 1] == "tiny"
    assert cmd[cmd.index("--reserve") + 1] == "7" and "--no-cpu-baseline" in cmd
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
