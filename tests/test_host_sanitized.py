"""The host planner built with AddressSanitizer, UndefinedBehaviorSanitizer
and the plan validator, driven over the workloads, random packed metadata
and argument errors (CPU only; see sanitize_host.py)."""
import os
import shutil
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_host_planner_under_sanitizers():
    sys.path.insert(0, HERE)
    import sanitize_host

    lib = sanitize_host.build()
    env = dict(os.environ)
    env["LD_PRELOAD"] = sanitize_host.runtime_preload()
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    r = subprocess.run([sys.executable, os.path.join(HERE, "sanitize_host.py"), "run", lib], env=env,
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert "plans valid" in r.stdout
