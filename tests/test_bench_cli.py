"""Host-side checks of bench.py's contract (no GPU): the one-GPU refusal, the
kernel naming the profiles use, and the rule that committed traffic counters
apply only to the kernel source they were taken on."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and "--gpus 2" in r.stderr
    assert r.stdout == ""


def test_kernel_names():
    assert bench.kernel_name("kv_fwd", 128) == "correct_h0_fwd_dma_kernel<128, 0>"
    assert bench.kernel_name("vk_fwd", 64) == "correct_h0_fwd_dma_kernel<64, 1>"
    assert bench.kernel_name("vk_bwd", 128) == "correct_h0_kernel<128, 1, 1>"
    assert bench.kernel_name("kv_fwd", 256) == "correct_h0_kernel<256, 0, 0>"


def test_source_hash_ignores_comments(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("int a; // note\n/* block\n comment */\nint b;\n\n")
    monkeypatch.setattr(bench, "KERNEL_SRC", str(src))
    h1 = bench.kernel_source_hash()
    src.write_text("int a; // other note\n\nint b;\n")
    assert bench.kernel_source_hash() == h1
    src.write_text("int a;\nint c;\n")
    assert bench.kernel_source_hash() != h1
    assert len(h1) == 16 and all(ch in "0123456789abcdef" for ch in h1)


def test_traffic_only_for_matching_source(tmp_path, monkeypatch):
    f = tmp_path / "traffic.md"
    f.write_text("Kernel source sha256[:16] (code only): `0123456789abcdef`\n\n"
                 "HBM bytes per launch (scaled), `correct_h0_fwd_dma_kernel<128, 0>`: 5.25e+07\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0123456789abcdef")
    assert bench.read_traffic("correct_h0_fwd_dma_kernel<128, 0>") == pytest.approx(5.25e7)
    assert bench.read_traffic("correct_h0_fwd_dma_kernel<128, 1>") is None
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "fedcba9876543210")
    assert bench.read_traffic("correct_h0_fwd_dma_kernel<128, 0>") is None
