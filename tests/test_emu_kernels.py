"""The library's kernels run on the CPU under AddressSanitizer, checked against the oracle.

tests/emu/build_emu.py compiles the HIP sources as host C++ against a small emulation of the
device (tests/emu: one fiber per GPU thread, workgroup barriers, 64-lane wave operations, the
DPP and lane-swap moves and an OCP E4M3FN model of v_mfma_f32_16x16x128_f8f6f4).  A selection of
the GPU parity tests then runs in a child process against that build, with uninitialised
memory and LDS filled with garbage.  This catches, without a GPU:
  * any out-of-bounds access of a kernel (global memory, LDS, host rows);
  * a barrier or wave operation reached by only part of a workgroup or wave;
  * reads of LDS or workspace memory that the step did not write first;
  * results that depend on the order in which workgroups, or the waves of a workgroup, run
    (they run in a seeded random order here);
  * (second test, ThreadSanitizer build) memory that two waves of one workgroup share without a
    barrier in between;
  * any result that differs from the oracle on the tests' own inputs.
It does not model concurrency between workgroups or memory ordering; those stay with the GPU
tests.  Skipped when clang's AddressSanitizer runtime is not installed.
"""

import os
import re
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
sys.path.insert(0, os.path.join(HERE, "emu"))
import build_emu  # noqa: E402

ASAN = build_emu.asan_runtime()
pytestmark = pytest.mark.skipif(ASAN is None, reason="clang AddressSanitizer runtime not found")

# The small and medium GPU parity cases; the full-size workloads take too long on one core.
SELECTION = [
    "tests/test_gpu_scores.py", "tests/test_gpu_topk.py", "tests/test_gpu_pool.py",
    "tests/test_gpu_decode.py", "tests/test_gpu_prefill.py", "tests/test_gpu_multistep.py",
    "tests/test_gpu_interquery.py", "tests/test_gpu_layers.py", "tests/test_gpu_fused.py",
    "tests/test_gpu_stress.py",
    "-k", "not full and not b8_64k and not b32 and not 32k and not topk_rows_exact "
          "and not 150000 and not 300000 and not small_exact[1000] and not prefill_chunk_loop "
          "and not 61_layers",
]


def _run_selection(tmp_path, lib, runtime, extra_env, selection):
    env = dict(os.environ)
    env.update(ECHO_EMU_LIB=lib, LD_PRELOAD=runtime,
               PYTHONPATH=os.pathsep.join([os.path.join(HERE, "emu"), ROOT]), **extra_env)
    log = tmp_path / "emu.log"
    with open(log, "w") as fh:
        r = subprocess.run([sys.executable, "-m", "pytest", "-p", "emu_plugin", "-p", "no:cacheprovider",
                            "-q", "-s", *selection], cwd=ROOT, env=env, stdout=fh,
                           stderr=subprocess.STDOUT, timeout=900)
    text = log.read_text()
    return r.returncode, text


def test_kernels_on_cpu_under_address_sanitizer(tmp_path):
    lib = build_emu.build(out=os.path.join(ROOT, "_build", "emu"))
    rc, text = _run_selection(
        tmp_path, lib, ASAN,
        dict(ECHO_EMU_ORDER="1",
             ASAN_OPTIONS="detect_leaks=0:detect_odr_violation=0:alloc_dealloc_mismatch=0:"
                          "detect_stack_use_after_return=0:abort_on_error=1"),
        ["-x", *SELECTION])
    assert rc == 0, text[-6000:]
    m = re.search(r"(\d+) passed", text)
    assert m and int(m.group(1)) >= 30, text[-3000:]


TSAN = build_emu.sanitizer_runtime("tsan")


@pytest.mark.skipif(TSAN is None, reason="clang ThreadSanitizer runtime not found")
def test_kernels_on_cpu_under_thread_sanitizer(tmp_path):
    """The waves of a workgroup are ThreadSanitizer fibers and its barriers are the only
    ordering between them, so any LDS or global location that two waves of one workgroup use
    without a barrier in between (unless both use atomics) is reported.  BLAS and torch run on
    one thread here: their own threads are not instrumented."""
    lib = build_emu.build(out=os.path.join(ROOT, "_build", "emu_tsan"), sanitizer="thread")
    rc, text = _run_selection(
        tmp_path, lib, TSAN,
        dict(ECHO_EMU_ORDER="2", OPENBLAS_NUM_THREADS="1", OMP_NUM_THREADS="1",
             TSAN_OPTIONS="halt_on_error=0:report_signal_unsafe=0"),
        SELECTION)
    races = text.count("WARNING: ThreadSanitizer")
    assert races == 0, text[text.index("WARNING: ThreadSanitizer"):][:6000]
    assert rc == 0, text[-6000:]
    m = re.search(r"(\d+) passed", text)
    assert m and int(m.group(1)) >= 30, text[-3000:]
