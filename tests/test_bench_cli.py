"""The bench's command-line contract on the host: it measures one GPU and says
so when asked for more, before touching any device."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_bench_lists_its_workloads():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--help"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0
    for wl in ("decode", "train", "offload", "prefill"):
        assert wl in r.stdout


def test_bench_rejects_an_unknown_workload():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workloads", "decode,decod"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "decod" in r.stderr and r.stdout == ""
