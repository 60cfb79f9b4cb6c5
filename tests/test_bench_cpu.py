"""Host-side contract of bench.py (no GPU): the one-GPU refusal, the algorithmic work the
roofline divides by, and the rule that the committed traffic figure is reported only for
the GEMM source it was measured on."""
import hashlib
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from mixture_experts_layer_46_amd import accounting as A  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stdout + r.stderr


def test_worked_shape_algorithmic_work_by_hand():
    # 8192 tokens, hidden 4096, 64 experts (all touched), top-2, SiLU two-layer FFN to 16384, bf16
    T, H, E, k, F = 8192, 4096, 64, 2, 16384
    P = T * k
    sb = A.stage_bytes(T, H, E, k, F, "silu2", "bf16", touched=64)
    # algorithmic: the first projection every expert's W1 once and x once, the second
    # every W2 once and out once
    assert sb.ffn_up == 64 * 4096 * 16384 * 2 + 8192 * 4096 * 2 == 8657043456
    assert sb.ffn_down == 64 * 16384 * 4096 * 2 + 8192 * 4096 * 2
    assert sb.ffn_up + sb.ffn_down == sb.layer
    # as designed: + h written once; + h read once and the y rows written once
    assert sb.ffn_up_designed == sb.ffn_up + 16384 * 16384 * 2 == 9193914368
    assert sb.ffn_down_designed == 64 * 16384 * 4096 * 2 + 16384 * 16384 * 2 + 16384 * 4096 * 2
    # 2 flops per multiply-add, one matrix each way
    assert A.ffn_up_flops(T, k, H, F, "silu2") == 2 * P * H * F == 2199023255552
    assert A.ffn_down_flops(T, k, H, F) == 2 * P * F * H
    # the whole layer: all weights once, x read and out written
    assert sb.layer == 2 * 64 * 4096 * 16384 * 2 + 2 * 8192 * 4096 * 2


def _summary(tmp_path, digest, kernel, up_bytes):
    (tmp_path / "profiles").mkdir()
    (tmp_path / "mixture_experts_layer_46_amd" / "csrc").mkdir(parents=True)
    src = tmp_path / "mixture_experts_layer_46_amd" / "csrc" / "grouped_gemm.hip"
    src.write_bytes(b"// kernel source\n")
    real = hashlib.sha256(src.read_bytes()).hexdigest()
    (tmp_path / "profiles" / "traffic_w.txt").write_text(
        "# summary\n"
        f"grouped_gemm.hip sha256: {real if digest is None else digest}\n"
        f"up kernel: {kernel}\n"
        f"up hbm bytes per launch: {up_bytes}\n")


def test_traffic_only_for_the_measured_source(tmp_path, monkeypatch):
    kern = "k_grouped_gemm_lds<320, 320, 1, 1, true>"
    _summary(tmp_path, None, kern, 123456789)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench._traffic("w", "up", kern) == pytest.approx(123456789)
    # another kernel than the one measured, or a workload with no summary: no figure
    assert bench._traffic("w", "up", "k_grouped_gemm_pp<256, 2, 1, true, false>") is None
    assert bench._traffic("other", "up", kern) is None


def test_traffic_dropped_once_the_source_changes(tmp_path, monkeypatch):
    kern = "k_grouped_gemm_lds<320, 320, 1, 1, true>"
    _summary(tmp_path, "0" * 64, kern, 123456789)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench._traffic("w", "up", kern) is None
