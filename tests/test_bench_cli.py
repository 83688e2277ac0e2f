"""bench.py's command-line contract, checked on the CPU (no GPU needed)."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_power_sampling_degrades_to_none_without_a_device():
    # The power / clock figures are context: where amdsmi or the device is
    # unavailable they are None and the benchmark goes on.
    code = ("import sys; sys.path.insert(0, %r); import bench; ps = bench.PowerSampler(); "
            "print(ps.smi is None, ps.run(lambda: None), bench.mfma_ceiling(print, ps))" % ROOT)
    r = subprocess.run([sys.executable, "-c", code], stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    assert r.stdout.strip().splitlines()[-1] == "True None None"
