"""Machine-code check of the producer kernels' step barriers (CPU only).

The producer waves of the K <= 128 kernels (both directions) copy M_{s+1} into LDS with 16-byte
LDS-DMA loads and then issue 4-byte LDS-DMA L2 warm-up loads for later steps.
At the step barrier they wait with ``s_waitcnt vmcnt(N)``, N being the number
of warm-ups just issued, and leave those outstanding.  Vector-memory counts
retire in issue order, so the wait covers every load issued before the N
newest -- which is correct only if the N newest vector-memory instructions
before the barrier are warm-ups and no copy of M comes after them.  The
compiler schedules the code, so this test reads the machine code of the built
libraries (the gfx950 code object inside each .so, disassembled with ROCm's
llvm-objdump) and checks the order at every such barrier of every producer
kernel.
"""
from __future__ import annotations

import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "linear_attention_context_amd")
LIBS = ["libqla.so", "libqla_delay.so"]
LLVM = "/opt/rocm/llvm/bin"
TARGET = "hipv4-amdgcn-amd-amdhsa--gfx950"

COPY = re.compile(r"^buffer_load_dwordx4\b.*\blds\b")
WARM = re.compile(r"^buffer_load_dword\s.*\blds\b")
VMEM = re.compile(r"^(buffer_|global_)")
# kernels with producer waves: the plain and variable-length K <= 128 kernels of
# both directions, and the grouped kernel at K <= 128 (mangled names)
K_DMA = (16, 32, 48, 64, 80, 96, 112, 128)
# and the two-tile kernels (plain, variable-length and grouped) at K a multiple of 32
K_PAIR = tuple(k for k in K_DMA if k % 32 == 0)
PRODUCER_KERNELS = re.compile(r"correct_h0_(fwd|bwd)_dma|correct_h0_pair_kernel|correct_h0_grouped_kernelILi(%s)E"
                              r"|correct_h0_grouped_pair_kernel|correct_h0_pair_varlen_kernel" % "|".join(map(str, K_DMA)))


def _tools():
    need = [shutil.which("objcopy"), os.path.join(LLVM, "clang-offload-bundler"), os.path.join(LLVM, "llvm-objdump")]
    if need[0] is None or not all(os.path.exists(t) for t in need[1:]):
        # the libraries are built (checked by the caller): their order cannot go unchecked
        pytest.fail("objcopy / clang-offload-bundler / llvm-objdump not available to check the built code")
    return need


def _disassemble(lib: str, tmp_path) -> str:
    objcopy, bundler, objdump = _tools()
    fat = tmp_path / "fatbin.bin"
    code = tmp_path / "gfx950.o"
    subprocess.run([objcopy, f"--dump-section=.hip_fatbin={fat}", lib, str(tmp_path / "stripped.so")],
                   check=True, capture_output=True)
    subprocess.run([bundler, "--type=o", f"--targets={TARGET}", f"--input={fat}", f"--output={code}", "--unbundle"],
                   check=True, capture_output=True)
    out = subprocess.run([objdump, "-d", "--no-show-raw-insn", str(code)], check=True, capture_output=True, text=True)
    return out.stdout


def _kernels(text: str):
    """(symbol, instruction list) of every producer kernel."""
    cur, body = None, []
    for raw in text.splitlines():
        m = re.match(r"^[0-9a-f]+ <(\S+)>:$", raw)
        if m:
            if cur is not None:
                yield cur, body
            cur, body = (m.group(1), []) if PRODUCER_KERNELS.search(m.group(1)) else (None, [])
            continue
        if cur is not None:
            ins = raw.split("//")[0].strip()
            if ins:
                body.append(ins)
    if cur is not None:
        yield cur, body


def _check(body):
    """Number of barriers checked, list of problems."""
    checked, problems = 0, []
    for i, ins in enumerate(body):
        m = re.match(r"^s_waitcnt vmcnt\((\d+)\)$", ins)
        if not m or i + 1 >= len(body) or body[i + 1] != "s_barrier":
            continue
        n = int(m.group(1))
        if n == 0:
            continue
        checked += 1
        # vector-memory instructions since the previous barrier, newest first
        since = []
        for j in range(i - 1, -1, -1):
            if body[j] == "s_barrier":
                break
            if VMEM.match(body[j]):
                since.append(body[j])
        newest, older = since[:n], since[n:]
        if len(newest) < n or not all(WARM.match(x) for x in newest):
            problems.append(f"vmcnt({n}) at instruction {i}: newest {newest}")
        if not any(COPY.match(x) for x in older):
            problems.append(f"vmcnt({n}) at instruction {i}: no copy of M before the warm-ups")
    return checked, problems


@pytest.mark.parametrize("name", LIBS)
def test_producer_barriers_cover_every_copy(name, tmp_path):
    lib = os.path.join(PKG, name)
    if not os.path.exists(lib):
        pytest.skip(f"{name} is not built")
    kernels = list(_kernels(_disassemble(lib, tmp_path)))
    # {fwd, bwd} x {kv, vk} x {plain, variable-length} at each K <= 128, and the grouped kernel there;
    # {fwd, bwd} x {kv, vk} x {plain, variable-length} two-tile kernels and the grouped two-tile kernel
    # at each K that is a multiple of 32
    assert len(kernels) == 9 * len(K_DMA) + 9 * len(K_PAIR), [k for k, _ in kernels]
    for sym, body in kernels:
        checked, problems = _check(body)
        # the barrier after the first copy and the one in the step loop, at least
        assert checked >= 2, (sym, checked)
        assert not problems, (sym, problems)


def test_checker_flags_a_copy_after_the_warmups():
    """The checker itself: a copy scheduled after a warm-up is reported."""
    good = ["buffer_load_dwordx4 v0, s[0:3], 0 offen lds", "buffer_load_dwordx4 v1, s[0:3], 0 offen lds",
            "buffer_load_dword v2, s[4:7], 0 offen lds", "buffer_load_dword v3, s[8:11], 0 offen lds",
            "s_waitcnt vmcnt(2)", "s_barrier"]
    assert _check(good) == (1, [])
    bad = good[:1] + [good[2], good[1], good[3]] + good[4:]
    checked, problems = _check(bad)
    assert checked == 1 and problems
