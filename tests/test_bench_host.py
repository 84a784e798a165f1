"""Host-side checks of bench.py: the one-GPU contract, the algorithmic byte counts the
roofline divides by, and the rule that a counter summary only counts while the kernel
sources still hash to the value it records."""
import hashlib
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.mark.parametrize("name,expected", [
    ("qwen35_0p8b_prefill_T4096", 85.5e6),
    ("qwen35_4b_prefill_B4_T16384", 2.17e9),
    ("qwen38_27b_prefill_T262144", 11.9e9),
])
def test_algorithmic_bytes(name, expected):
    B, T, Hk, Hv = bench.WORKLOADS[name]
    got = bench.prefill_bytes(B, T, Hk, Hv)
    assert abs(got / expected - 1) < 0.01
    # per token: q, k (Hk heads) + v, z, o (Hv heads) in bf16, g and beta in fp32
    per_tok = 2 * Hk * 128 * 2 + 3 * Hv * 128 * 2 + Hv * 8
    assert got >= B * T * per_tok


def test_tiny_case_reads_no_conv_or_gate():
    B, T, Hk, Hv = bench.WORKLOADS["tiny_T64"]
    assert bench.prefill_bytes(B, T, Hk, Hv, fused=False) == T * (2 * 128 * 2 + 2 * 128 * 2 + 8) + 128 * 128 * 4


def test_headline_is_the_27b_shaped_layer():
    assert bench.HEADLINE == "qwen38_27b_prefill_T262144"
    assert bench.WORKLOADS[bench.HEADLINE] == (1, 262144, 16, 48)


def _summary(tmp_path, sources, digest):
    p = tmp_path / "summary.txt"
    p.write_text("header line without the fields\n"
                 "traffic_bytes_per_call: 123456789\n"
                 "mfma_issued_flop_per_call: 1.5e12\n"
                 f"sources_sha256: {digest}\n"
                 f"sources: {' '.join(sources)}\n")
    return p


def test_counter_summary_follows_the_sources(tmp_path, monkeypatch):
    src = os.path.join(ROOT, "gated_deltanet_mixer_amd/csrc/gdn_pass.hip")
    h = hashlib.sha256(open(src, "rb").read()).hexdigest()
    good = _summary(tmp_path, [src], h)
    monkeypatch.setitem(bench.COUNTER_FILES, "x", str(good))
    monkeypatch.setattr(bench, "ROOT", "/")
    got = bench.measured_counters("x")
    assert got["traffic"] == 123456789 and got["mfma_issued_flop_per_call"] == 1.5e12
    stale = _summary(tmp_path, [src], "0" * 64)
    monkeypatch.setitem(bench.COUNTER_FILES, "x", str(stale))
    assert bench.measured_counters("x") is None
    assert bench.measured_counters("no_such_workload") is None
