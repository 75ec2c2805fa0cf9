"""The benchmark's command-line contract and its link to the committed
profiles, checked without a GPU."""
import hashlib
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_profiled_run_flags_parse(monkeypatch):
    monkeypatch.setattr(sys, "argv", ["bench.py", "--steps", "20", "--warmup", "5", "--no-graph",
                                      "--no-kernel-timer", "--copy-calibration"])
    a = bench.parse()
    assert (a.steps, a.warmup, a.no_graph, a.no_kernel_timer, a.copy_calibration) == (20, 5, True, True, True)
    monkeypatch.setattr(sys, "argv", ["bench.py"])
    a = bench.parse()
    assert a.gpus == 1 and a.steps > 0 and a.warmup > 0 and not a.no_kernel_timer


@pytest.mark.parametrize("name", sorted(f[:-3] for f in os.listdir(os.path.join(ROOT, "profiles"))
                                        if f.endswith(".md")))
def test_committed_profiles_match_the_kernel_sources(name):
    """Each profile summary records a hash of the kernel source it measured
    (with device_common.h); a kernel change without a new profile fails here."""
    txt = open(os.path.join(ROOT, "profiles", name + ".md")).read()
    m = re.search(r"kernel_source_sha256:\s*([0-9a-f]+)", txt)
    assert m, "profile without a source hash"
    src_file = {"gemv": "gemv.hip", "skinny": "mfma_gemv.hip", "mfma": "gemm_mfma.hip",
                "huffman": "decode.hip"}[name.split("_")[0]]
    csrc = os.path.join(ROOT, "mlp_matmul_amd", "csrc")
    src = open(os.path.join(csrc, src_file), "rb").read() + open(os.path.join(csrc, "device_common.h"), "rb").read()
    assert hashlib.sha256(src).hexdigest()[:16] == m.group(1)[:16]
    assert "rocprofv3" in txt


def test_headline_traffic_comes_from_the_current_profile():
    t = bench.traffic_from_profiles("gemv_gateup_pal_llama_mlp_b1")
    assert t is not None and 1.7e8 < t < 2.0e8     # ~180 MB read per fused gate/up launch
