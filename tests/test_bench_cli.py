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
    """The names rocprofv3 reports for the kernels each variant launches."""
    assert bench.kernel_name("kv_fwd", 128) == "correct_h0_fwd_dma_kernel<128, 0>"
    assert bench.kernel_name("vk_fwd", 64) == "correct_h0_fwd_dma_kernel<64, 1>"
    assert bench.kernel_name("vk_bwd", 128) == "correct_h0_bwd_dma_kernel<128, 1>"
    assert bench.kernel_name("kv_bwd", 48) == "correct_h0_bwd_dma_kernel<48, 0>"
    assert bench.kernel_name("kv_fwd", 256) == "correct_h0_kernel<0, 0, false>"
    assert bench.kernel_name("vk_bwd", 256) == "correct_h0_kernel<1, 1, false>"
    assert bench.kernel_name("kv_bwd", 192) == "correct_h0_kernel<0, 1, true>"


def test_kernel_names_match_the_built_library():
    """Every name kernel_name() gives for the 32K x 32-head step and the wide
    configuration is a kernel the built library contains (mangled)."""
    import re
    lib = os.path.join(ROOT, "linear_attention_context_amd", "libqla.so")
    if not os.path.exists(lib):
        pytest.skip("libqla.so is not built")
    data = open(lib, "rb").read()
    for v in ("kv_fwd", "vk_fwd", "kv_bwd", "vk_bwd"):
        for K in (128, 256, 192):
            name = bench.kernel_name(v, K)
            base, targs = re.match(r"(\w+)<(.*)>", name).groups()
            parts = [t.strip() for t in targs.split(",")]
            mangled = "".join("Lb0E" if t == "false" else "Lb1E" if t == "true" else f"Li{t}E" for t in parts)
            assert (base + "I" + mangled).encode() in data, name


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
