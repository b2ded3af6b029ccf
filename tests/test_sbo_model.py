"""CPU model of the single-batch-overlap protocol (signalled down GEMM ->
polling combine; DeepGEMM single-batch-overlap pull request, sections 2-3)
under ThreadSanitizer: the protocol as the kernels implement it runs clean,
and the same model with the consumer's wait removed is reported."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "sbo_model", "sbo_model.c")
ENV = dict(os.environ, TSAN_OPTIONS="halt_on_error=1 exitcode=66")


def _build(tmp_path, broken):
    exe = str(tmp_path / ("sbo_broken" if broken else "sbo_model"))
    cmd = ["gcc", "-O1", "-g", "-fsanitize=thread", "-pthread"] + (["-DBROKEN"] if broken else []) + [SRC, "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        pytest.skip("no ThreadSanitizer toolchain: " + r.stderr[-300:])
    return exe


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_sbo_protocol_is_race_free(tmp_path):
    exe = _build(tmp_path, broken=False)
    orphans = 0
    for seed in range(1, 6):
        r = subprocess.run([exe, str(seed)], capture_output=True, text=True, env=ENV, timeout=120)
        assert r.returncode == 0, r.stdout + r.stderr[-2000:]
        assert "mismatches 0" in r.stdout
        orphans += int(r.stdout.split("orphans")[1].split()[0])
    assert orphans > 0  # the second pass (tokens with no local row) ran


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_sbo_model_detects_a_missing_wait(tmp_path):
    exe = _build(tmp_path, broken=True)
    r = subprocess.run([exe, "3"], capture_output=True, text=True, env=ENV, timeout=120)
    assert r.returncode == 66 and "data race" in r.stderr
