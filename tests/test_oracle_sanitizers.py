"""The C oracle under the compiler's sanitizers (CPU only).

tests/sanitize/oracle_runner.c runs every oracle entry (the plain step, top-p,
top-k with top-p, candidate trees, prompt lookup) on small seeded batches with
ragged lengths, greedy and sampling sequences and planted input errors. It is
built with gcc twice: AddressSanitizer + UndefinedBehaviorSanitizer (any
finding aborts), and ThreadSanitizer with the batch split over threads, as the
Python wrapper runs it.
"""
import os
import shutil
import subprocess

import pytest

from conftest import ROOT

SRC = [os.path.join(ROOT, "oracle", "spec_verify_ref.c"),
       os.path.join(ROOT, "tests", "sanitize", "oracle_runner.c")]
BASE = ["gcc", "-O1", "-g", "-std=c11", "-ffp-contract=off", "-fno-omit-frame-pointer"]

pytestmark = pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")


def _build_and_run(tmp_path, name, flags, threads, env_extra):
    exe = str(tmp_path / name)
    build = subprocess.run(BASE + flags + ["-o", exe] + SRC + ["-lm", "-lpthread"],
                           capture_output=True, text=True)
    if build.returncode != 0 and "sanitize" in build.stderr:
        pytest.skip(f"gcc here cannot build with {flags}: {build.stderr[-300:]}")
    assert build.returncode == 0, build.stderr
    env = dict(os.environ, **env_extra)
    run = subprocess.run([exe, str(threads)], capture_output=True, text=True, env=env,
                         timeout=300)
    assert run.returncode == 0, run.stdout + run.stderr[-4000:]
    assert "oracle runner: ok" in run.stdout


def test_oracle_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    _build_and_run(tmp_path, "asan", ["-fsanitize=address,undefined",
                                      "-fno-sanitize-recover=all"], 1,
                   {"ASAN_OPTIONS": "detect_leaks=1:abort_on_error=1:verify_asan_link_order=0",
                    "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1"})


def test_oracle_threads_under_thread_sanitizer(tmp_path):
    _build_and_run(tmp_path, "tsan", ["-fsanitize=thread"], 4,
                   {"TSAN_OPTIONS": "halt_on_error=1"})
