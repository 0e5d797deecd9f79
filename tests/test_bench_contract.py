"""CPU checks of bench.py's command-line contract that need no GPU: more than one GPU is refused with a
message and a non-zero status before anything touches a device, and the headline workload is named."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=300, cwd=ROOT)
    assert r.returncode != 0
    assert "--gpus 2 is not supported" in r.stderr and "one GPU" in r.stderr
    assert r.stdout.strip() == ""  # no JSON line


def test_workloads_are_chosen_by_name():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--config", "3"], capture_output=True,
                       text=True, timeout=300, cwd=ROOT)
    assert r.returncode != 0 and "invalid choice" in r.stderr
