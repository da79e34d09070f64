"""The library's host code (tq_host.cpp: codebook solvers, layer randomness,
page descriptors, sizing, validation and its per-thread messages) built for the
CPU with the address and undefined-behaviour sanitizers, and again with the
thread sanitizer, and driven by tests/host_sanitize_driver.cpp: valid calls
(checked against properties that hold by definition), invalid ones (which must
fail cleanly) and eight host threads calling at once.  Plain g++; no GPU code
is built here."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "kv_cache_vector_srht_amd", "csrc", "tq_host.cpp")
DRIVER = os.path.join(ROOT, "tests", "host_sanitize_driver.cpp")
INC = [os.path.join(ROOT, "include"), os.path.join(ROOT, "kv_cache_vector_srht_amd", "csrc")]


@pytest.mark.parametrize("sanitizers", ["address,undefined", "thread"])
def test_host_code_under_sanitizers(tmp_path, sanitizers):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("no g++")
    exe = str(tmp_path / "driver")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", f"-fsanitize={sanitizers}",
           "-fno-sanitize-recover=all", *[f"-I{d}" for d in INC], SRC, DRIVER, "-o", exe, "-pthread"]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", TSAN_OPTIONS="halt_on_error=1")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all checks passed" in r.stdout
