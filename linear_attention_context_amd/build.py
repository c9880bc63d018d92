"""Build libqla.so (the C-ABI library with the gfx950 kernels) in-tree with hipcc.

``python -m linear_attention_context_amd.build`` or ``build()`` from Python.
Always recompiles when called; the result lands next to this file as
``libqla.so`` (plus ``libqla_delay.so``, the same library with a forced-delay
schedule compiled in, used by the race tests).
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
SOURCES = [os.path.join(CSRC, "qla_api.cpp"), os.path.join(CSRC, "qla_kernels.hip")]
LIB = os.path.join(PKG, "libqla.so")
LIB_DELAY = os.path.join(PKG, "libqla_delay.so")
ARCH = "gfx950"

# Packed fp32 VALU instructions are kept out of the device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc_command(out: str, defines=()) -> list:
    cmd = ["hipcc", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Wall", "-Werror", "-fvisibility=hidden", "-Wno-unused-command-line-argument",
           f"-I{INCLUDE}", f"-I{CSRC}", *DEVICE_FLAGS]
    cmd += [f"-D{d}" for d in defines]
    cmd += ["-o", out, *SOURCES]
    return cmd


def _start(out: str, defines=()):
    tmp = out + f".tmp{os.getpid()}"
    proc = subprocess.Popen(hipcc_command(tmp, defines), stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)
    return out, tmp, proc


def _finish(job) -> None:
    out, tmp, proc = job
    _, stderr = proc.communicate()
    # The host pass reports the device-only feature flag as unknown; that line is expected.
    noise = "'-packed-fp32-ops' is not a recognized feature for this target"
    err = "\n".join(l for l in stderr.splitlines() if noise not in l)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed for {out}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    os.replace(tmp, out)


def build() -> str:
    # the two libraries compile in parallel
    jobs = [_start(LIB), _start(LIB_DELAY, defines=("QLA_DEBUG_DELAY=1",))]
    for job in jobs:
        _finish(job)
    return LIB


if __name__ == "__main__":
    print(build())
