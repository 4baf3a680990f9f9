"""bench.py's argument checks, which run before anything touches a GPU:
one GPU only, and the layout, rotation and slot-pool options."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120)


@pytest.mark.parametrize("args,needle", [
    (["--gpus", "2"], "only one GPU"),
    (["--gpus", "8", "--steps", "3"], "only one GPU"),
    (["--stagger", "100"], "--stagger 100"),
    (["--stagger", "-256"], "--stagger -256"),
    (["--slot-stream", "--slots", "1"], "--slots 1"),
    (["--state-sets", "-1"], "--state-sets -1"),
])
def test_refused_before_any_gpu_work(args, needle):
    r = bench(*args)
    assert r.returncode == 2, r.stderr
    assert needle in r.stderr
    assert r.stdout == ""          # no JSON line


def test_help_lists_the_workloads_and_options():
    r = bench("--help")
    assert r.returncode == 0
    for word in ("--workload", "--stagger", "--slots", "--state-sets", "--q8", "--slot-stream",
                 "--merge"):
        assert word in r.stdout
