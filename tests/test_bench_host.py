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


def test_one_line_fits_a_2000_character_tail():
    # a reader that keeps the last 2000 characters of the output gets the whole line, with
    # every section present at realistic sizes
    dec = {"workload": "b64_128k", "prefetch": "ranged", "us_per_step": 1979.61,
           "indexed_tokens_per_s": 4237522077.01, "scoring_frac": 0.61631, "recall_frac_of_link": 0.97512,
           "memcpy_recall_us": 272037.12, "prefetch_modes": {m: {"us": 2018.25, "n_miss": 63907,
                                                                  "prefetched": 8192}
                                                              for m in ("off", "ranged", "fused")}}
    out = {"metric": bench.METRIC, "value": 4873318709.21, "unit": "indexed tokens/s", "n_gpus": 1,
           "steps": 50, "warmup": 5, "ms_per_step": 0.10758, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "fp8_e4m3 (fp32 accumulate)",
           "data": "synthetic (seeded)",
           "config": {"workload": "b8_64k", "description": "x" * 200, "batch": 8, "tokens": 524288,
                      "topk": 2048, "n_gpu_slots": 65536, "n_host_slots": 524288, "prefetch": "off",
                      "free_slots_at_start": 0, "timing": "y" * 200},
           "roofline": {"bound": "hbm", "kernel": "z" * 120, "achieved": 4730.81, "peak": 8000.0,
                        "unit": "GB/s", "frac": 0.59131, "traffic": 69933070,
                        "bytes_per_launch": 67108864, "us_per_launch": 14.19, "plain_scoring_us": 12.95},
           "step": {"hbm_frac": 0.078, "link_floor_us": 33.0, "scoring_floor_us": 8.4},
           "recall": {"achieved": 47.61, "peak_measured_h2d": 57.17, "frac": 0.83261, "rows": 1640,
                      "memcpy_baseline_us_median": 7009.01, "kernel": "recall_gather_kernel"},
           "breakdown_us": {"step": 107.58}, "counters": {"n_miss": 1640},
           "cpu_baseline": {"value": 2496858.9, "unit": "indexed tokens/s", "cores": 16,
                            "cpu_model": "AMD EPYC 9575F 64-Core Processor (128 cores online)",
                            "kind": "oracle", "seconds": 10.079,
                            "sample": "48 x the whole oracle decode step, 524288 tokens each (fp64 "
                                      "scores, exact top-k, pool step, recall copy)"}}
    extra = {"c3": dict(dec, workload="b32_ragged"), "c5": dec,
             "layers": {"us_per_model_step": 5431.81, "us_per_layer": 89.05},
             "prefill": {"frac": 0.46573, "achieved": 2328.61, "us_per_launch": 3777.51,
                         "topk_rows_us": 1518.61},
             "prefill_offload": {"pairs_per_s": 5255141194.31, "thr_bin_median_shifted": 2287,
                                 "thr_bin_median_unshifted": 4515},
             "loop": {"us_per_step_median": 384.61, "hit_rate_median": 0.9822,
                      "fused": {"us_per_step_median": 263.71}, "off": {"us_per_step_median": 193.01,
                                                                      "hit_rate_median": 0.8101}},
             "prefetch_modes": {m: {"us": 191.65, "n_miss": 1555, "prefetched": 512}
                                for m in ("off", "ranged", "fused")}}
    line = json.dumps(bench.one_line(out, extra))
    assert len(line) < 2000, len(line)
    d = json.loads(line)
    for key in ("metric", "value", "unit", "roofline", "cpu_baseline", "c5", "prefill", "loop"):
        assert key in d
    assert d["roofline"]["frac"] == 0.59131 and d["c5"]["modes_us"]["ranged"] == 2018.25
