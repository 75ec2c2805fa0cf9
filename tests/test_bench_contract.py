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
    a = bench.parse(["--steps", "20", "--warmup", "5", "--no-kernel-timer", "--copy-calibration", "--no-sweep",
                     "--no-cpu-baseline", "--no-compare"])
    assert (a.steps, a.warmup, a.no_kernel_timer, a.copy_calibration, a.no_sweep) == (20, 5, True, True, True)
    a = bench.parse([])
    assert a.gpus == 1 and a.steps > 0 and a.warmup > 0 and not a.no_kernel_timer
    assert a.layers == 32 and a.batch == 1 and a.min_warmup_ms >= 50


def test_headline_line_stays_compact():
    """The stdout line the benchmark prints, with every field at a realistic
    width, stays under 2 KB (the sweep detail goes to a file)."""
    line = {
        "metric": bench.METRIC, "value": 6666.6, "unit": "GB/s", "n_gpus": 1, "steps": 20, "warmup": 5,
        "warmup_steps_run": 120, "ms_per_step": 1.6912, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "llama3.1-8b-mlp-stack", "layers": 32, "batch": 1, "gate_up": [14336, 4096],
                   "down": [4096, 14336], "pipeline": "auto",
                   "plan": {"14336x4096": "direct/gemv", "4096x14336": "direct/gemv"}, "gate_up_fused": True,
                   "weights": "N(0,0.02)+U[0.01%,0.2%] N(0,0.5) outliers per layer, seeded"},
        "compressed_GBps": 5100.1, "compressed_hbm_frac": 0.6375, "bf16_ms_per_step": 1.9812,
        "speedup_vs_bf16": 1.1715, "sizes_GB": {"bf16": 11.27, "huffman": 7.78, "palette": 8.65},
        "verbatim_group_frac": 0.03093, "decode_bitexact": "96/96",
        "roofline": {"bound": "hbm", "achieved": 6200.1, "peak": 8000.0, "unit": "GB/s", "frac": 0.775,
                     "traffic": 181783460.0, "kernel": "fused gate/up + SiLU (direct palette)", "launches": 640,
                     "avg_launch_us": 28.951, "bytes_per_launch": 179530408,
                     "profile_avg_us": 30.039,
                     "all_matmuls_frac": 0.7391, "per_kind_avg_us": {"gate_up": 28.95, "down": 16.71}},
        "sweep": {"cols": "batch,ms,bf16_ms,x_bf16",
                  "rows": [[b, 1.6912, 1.9812, 1.1715] for b in (1, 2, 4, 8, 16, 32, 64, 128, 256)]},
        "cpu_baseline": {"value": 0.6512, "unit": "GB/s", "cores": 16, "kind": "oracle",
                         "sample": "stack layer 0, 1/16 of gate/up/down rows, B=1: 4-bit rebuild + fp64 matmul + "
                                   "SiLU, 33 reps/6.1 s; codec 1 thread, BLAS 16",
                         "stages_GBps": {f"c{i}": [0.0123, 0.0321, 0.0321, 0.0321, 0.123, 1.23] for i in range(1, 6)},
                         "stage_order": ",".join(bench.CPU_STAGES), "seconds": 31.2},
        "detail": "bench_out/bench_detail.json",
    }
    import json
    assert len(json.dumps(line, separators=(",", ":"), ensure_ascii=False).encode()) < 2000


@pytest.mark.parametrize("name", sorted(f[:-3] for f in os.listdir(os.path.join(ROOT, "profiles"))
                                        if f.endswith(".md")))
def test_committed_profiles_match_the_kernel_sources(name):
    """Each profile summary records a hash of the kernel source it measured
    (with device_common.h); a kernel change without a new profile fails here."""
    txt = open(os.path.join(ROOT, "profiles", name + ".md")).read()
    m = re.search(r"kernel_source_sha256:\s*([0-9a-f]+)", txt)
    assert m, "profile without a source hash"
    src_files = {"gemv": ["gemv.hip"], "skinny": ["mfma_gemv.hip", "skinny_dma.hip"], "mfma": ["gemm_mfma.hip", "gemm_lds.hip"],
                 "huffman": ["decode.hip"]}[name.split("_")[0]]
    csrc = os.path.join(ROOT, "mlp_matmul_amd", "csrc")
    src = b"".join(open(os.path.join(csrc, f), "rb").read() for f in src_files)
    src += open(os.path.join(csrc, "device_common.h"), "rb").read()
    assert hashlib.sha256(src).hexdigest()[:16] == m.group(1)[:16]
    assert "rocprofv3" in txt


def test_headline_traffic_comes_from_the_current_profile():
    traffic, avg_us = bench.profile_figures("gemv_gateup_pal_llama_mlp_stack_b1")
    assert traffic is not None and 1.7e8 < traffic < 2.0e8     # ~182 MB read per fused gate/up launch
    assert avg_us is not None and 20 < avg_us < 40
