"""Host logic of bench.py on the CPU: the algorithmic FLOP and byte counts
the roofline fractions divide by, the roofline bound they are taken
against, the refusal of more than one GPU, and the rule that a traffic
profile counts only while the GEMM source is unchanged."""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_algorithmic_counts_mixtral_prefill():
    w = workloads.WORKLOADS["mixtral_prefill"]
    counts = np.array([1005, 1005, 1049, 1018, 1041, 1070, 1014, 990])
    a = bench.algorithmic(w, counts, counts)
    rows = 8192
    # router 2 T d E + two expert GEMMs 2 rows d d_ff each
    assert a["flops"] == 2 * 4096 * 4096 * 8 + 4 * rows * 4096 * 14336
    assert a["up_flops"] == 2 * rows * 4096 * 14336
    # router weights + W1 and W2 of the 8 touched experts + x and y
    assert a["bytes"] == 8 * 4096 * 2 + 8 * 2 * 4096 * 14336 * 2 + 2 * 4096 * 4096 * 2
    # up GEMM: W1 once, the gathered rows, H
    assert a["up_bytes"] == 8 * 14336 * 4096 * 2 + rows * (4096 + 14336) * 2
    assert a["rows"] == rows and a["touched"] == 8


def test_algorithmic_counts_skip_untouched_experts_and_fp8():
    w = workloads.WORKLOADS["mixtral_decode_fp8"]
    kept = np.array([9, 0, 8, 8, 8, 8, 8, 15])        # expert 1 untouched
    a = bench.algorithmic(w, kept, kept)
    assert a["touched"] == 7 and a["rows"] == 64
    # E4M3 codes (1 byte) plus one fp32 scale per output channel
    assert a["up_bytes"] == 7 * 14336 * (4096 + 4) + 64 * (4096 + 14336) * 2
    w2 = workloads.WORKLOADS["deepseek_v3"]              # + shared expert
    kept2 = np.full(256, 256)
    a2 = bench.algorithmic(w2, kept2, kept2)
    assert a2["touched"] == 257 and a2["rows"] == 65536 + 8192


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"),
                        "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_profile_needs_the_current_gemm_source(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    # the digest is taken over the real sources
    digest = bench.source_digest()
    (prof / "gemm_up_x_hbm_traffic.txt").write_text(
        f"traffic_bytes_per_launch: 123\ngemm_source_sha256_16: {digest}\n")
    assert bench.recorded_traffic("x") == 123.0
    (prof / "gemm_up_y_hbm_traffic.txt").write_text(
        "traffic_bytes_per_launch: 123\ngemm_source_sha256_16: 0000\n")
    assert bench.recorded_traffic("y") is None
    assert bench.recorded_traffic("missing") is None


def test_roofline_bound_by_arithmetic_intensity():
    """The up GEMM's bound is the peak it would take longer at: the Mixtral
    prefill GEMM (775 FLOP per byte) is matrix-bound; the DeepSeek-shaped
    one (8192 x 8 + 8192 rows over 257 experts' weights: 243 FLOP per
    byte), the Expert-Choice one (181) and the decode one are HBM-bound,
    all against the 312 FLOP per byte of 2.5 PFLOP/s over 8 TB/s."""
    W = workloads.WORKLOADS
    peak = bench.MFMA_BF16_PEAK_TFLOPS
    cases = {"mixtral_prefill": (np.full(8, 1024), "mfma"),
             "deepseek_v3": (np.full(256, 256), "hbm"),
             "mixtral_decode": (np.full(8, 8), "hbm"),
             "mixtral_prefill_swiglu": (np.full(8, 1024), "mfma")}
    for name, (kept, want) in cases.items():
        a = bench.algorithmic(W[name], kept, kept)
        assert bench.roofline_bound(a, peak) == want, name
    ec = W["expert_choice_c2"]
    kept = np.full(ec.E, 256)
    a = bench.algorithmic(ec, kept, kept)
    assert 150 < a["up_flops"] / a["up_bytes"] < 312
    assert bench.roofline_bound(a, peak) == "hbm"
