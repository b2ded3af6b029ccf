"""bench.py's command line on the CPU: more than one GPU is refused with exit
code 2 before anything touches a device, and the defaults are one GPU, the
decode layer and a run of 5 + 20 steps."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_several_gpus_are_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "8"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "--gpus 8" in r.stderr and "one GPU" in r.stderr
    assert r.stdout == ""


def test_defaults(monkeypatch):
    sys.path.insert(0, ROOT)
    import bench
    monkeypatch.setattr(sys, "argv", ["bench.py"])
    a = bench.parse()
    assert (a.gpus, a.steps, a.warmup, a.workload, a.cpu_tokens) == (1, 20, 5, "decode_bf16", -1)
    assert not (a.graph or a.ue8m0 or a.tbo or a.calibrate_copy)
