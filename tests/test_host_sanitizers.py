"""The host half of the library (compressor, serialized format, validator,
plan table) built with AddressSanitizer and UndefinedBehaviorSanitizer by g++
and driven through its C entry points by tests/host_sanitize_driver.cpp:
ordinary, ragged and degenerate matrices, serialized images with flipped or
truncated bytes, and the plan file.  CPU only; skipped where g++ or the
sanitizer runtimes are missing."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mlp_matmul_amd", "csrc")
FLAGS = ["-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
         "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]


def _build(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not found")
    probe = tmp_path / "probe.cpp"
    probe.write_text("int main() { return 0; }\n")
    if subprocess.run([gxx, *FLAGS, str(probe), "-o", str(tmp_path / "probe")],
                      capture_output=True).returncode != 0:
        pytest.skip("sanitizer runtimes not available to g++")
    exe = tmp_path / "host_sanitize_driver"
    cmd = [gxx, *FLAGS, "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(ROOT, "tests", "host_sanitize_driver.cpp"),
           os.path.join(CSRC, "compress.cpp"), os.path.join(CSRC, "host_misc.cpp"),
           "-pthread", "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    return exe


def test_host_library_under_asan_ubsan(tmp_path):
    exe = _build(tmp_path)
    env = dict(os.environ,
               ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=600)
    out = r.stdout + r.stderr
    assert "runtime error" not in out, out[-4000:]
    assert "AddressSanitizer" not in out and "LeakSanitizer" not in out, out[-4000:]
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), out[-4000:]
