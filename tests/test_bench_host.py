"""Host logic of bench.py (no GPU): the grouped FFN's FLOP count against the
layer shapes, the one-GPU guard, and which counter summaries the bench line
may use."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from workloads import CONFIGS  # noqa: E402


@pytest.mark.parametrize("name,expected", [
    # dropless: every one of the T*k assignments is a grouped row; SwiGLU does
    # three d x d_ff products per row (gate, up, down), ReLU two
    ("tiny_fp32", 1.048576e6),          # 4 * 128 * 32 * 64
    ("small_bf16", 1.417e11),           # 6 * 8192 * 1024 * 2816
    ("mixtral_bf16", 5.772e12),         # 6 * 16384 * 4096 * 14336
    ("finegrained_bf16", 1.237e12),     # 6 * 131072 * 2048 * 768
])
def test_ffn_flops_matches_the_layer_shapes(name, expected):
    cfg = CONFIGS[name]
    got = bench.ffn_flops(cfg.T * cfg.k, cfg.d, cfg.d_ff, cfg.act)
    assert got == pytest.approx(expected, rel=1e-3)


def test_more_than_one_gpu_is_refused_before_any_device_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_counter_summaries_used_only_on_the_sources_they_were_taken_on(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    prof = tmp_path / "profiles"
    prof.mkdir()
    csrc = tmp_path / "grouped_expert_ffn_amd" / "csrc"
    csrc.mkdir(parents=True)
    for n in bench.FFN_SOURCES:
        (csrc / n).write_text(f"// {n}\n")
    sha = bench.kernel_source_sha()
    (prof / "pmc_grouped_ffn_w.txt").write_text(
        f"hbm_bytes_per_launch: 1.5e+09\nsource_sha: {sha}\n")
    (prof / "mfma_grouped_ffn_w.txt").write_text(f"gemm_clock_ghz: 1.81\nsource_sha: {sha}\n")
    assert bench.measured_traffic("w") == 1.5e9
    assert bench.measured_clock("w") == 1.81
    assert bench.measured_traffic("absent") is None
    # a kernel source changes: the summaries no longer describe the kernels
    (csrc / "ffn.hip").write_text("// ffn.hip, changed\n")
    assert bench.kernel_source_sha() != sha
    assert bench.measured_traffic("w") is None
    assert bench.measured_clock("w") is None
