"""The benchmark's host-side pieces without a GPU: the multi-GPU request is
refused with a message, and the committed counter summaries are read only
when they were taken on the current kernel sources."""
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "--gpus 1" in r.stderr
    assert r.stdout.strip() == ""


def test_kernel_source_sha_ignores_comments(tmp_path, monkeypatch):
    src = tmp_path / "weight_gradient_gemm_amd" / "csrc"
    src.mkdir(parents=True)
    for fn in bench.KERNEL_SOURCES:
        (src / fn).write_text("int a;\n// note\nint b; /* c */\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h1 = bench.kernel_source_sha()
    for fn in bench.KERNEL_SOURCES:
        (src / fn).write_text("int a;   \n\n// another note\nint b;\n")
    assert bench.kernel_source_sha() == h1
    (src / bench.KERNEL_SOURCES[0]).write_text("int a2;\nint b;\n")
    assert bench.kernel_source_sha() != h1


@pytest.fixture
def fake_profiles(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "pmc_w.txt").write_text(
        "# HBM-side byte counters: w\nkernel_source_sha: abc123\n"
        "fused_hbm_bytes_per_launch: 3.0e+09\nunfused_pair_hbm_bytes_per_step: 3.7e+09\n"
        "fused_write_bytes: 1.2e+09\n")
    (prof / "pmc_mfma_w.txt").write_text(
        "kernel_source_sha: abc123\n| kernel | dispatches | MFMA busy |\n|---|---|---|\n"
        "| fused AdamW (bf16 m,v, persistent) [epi 8] | 7 | 0.620 | 1.5e+06 |\n"
        "| fused AdamW (persistent) [epi 0] | 14 | 0.601 | 1.5e+06 | 900.0 | 1.80 | 3e+07 |\n"
        "| fused AdamW from fp8 inputs (X E4M3, dY E5M2, persistent) [epi 32] | 7 | 0.45 |\n"
        "| gradient (fp32 out, persistent) [epi 2] | 7 | 0.679 | 1.3e+06 |\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))


def test_counters_read_when_the_sources_match(fake_profiles):
    assert bench.read_traffic("w", "abc123") == 3.0e9
    c = bench.read_counters("w", "abc123", 100_000_000)
    assert c == {"fused_write_bytes_per_param": 12.0, "unfused_pair_hbm_bytes": 3.7e9,
                 "mfma_busy_fraction": 0.601, "profiled_clock_ghz": 1.8,
                 "from": "profiles/pmc_w.txt, pmc_mfma_w.txt (committed)"}


def test_counters_dropped_when_the_sources_changed(fake_profiles):
    assert bench.read_traffic("w", "other") is None
    assert bench.read_counters("w", "other", 100_000_000) is None
    assert bench.read_traffic("missing", "abc123") is None


def test_token_override_keeps_the_layer():
    import synth
    base = synth.CONFIGS[1]
    c = bench.with_tokens(base, 2048)
    assert (c.T, c.d_in, c.d_out, c.seed_base) == (2048, base.d_in, base.d_out, base.seed_base)
    assert c.name.endswith("_T2048") and "_T8192" not in c.name
