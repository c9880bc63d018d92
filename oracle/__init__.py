"""fp64 CPU oracle for the CP state-correction recurrence.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product path
(``linear_attention_context_amd``) never imports it and shares no code with it.

The arithmetic lives in ``qla_oracle.c`` (plain triple loops in fp64, contraction
index ascending); this module only marshals numpy arrays through ctypes and
compiles the C file with gcc when the shared object is missing.  The recurrence
it computes, and the page sections it follows, are stated in the C file's
header: the forward pass is S_j = M_j S_{j-1} + H_j, the backward pass
G_j = M_j^T G_{j+1} + H_j in reverse segment order (kv view), vk stores the
transposed state and multiplies on the right.

``correct_h0_varlen`` does no arithmetic of its own: it cuts packed ragged
chains (the variable-length case the correction note's performance section
benchmarks) out of their buffers and runs each through ``correct_h0``.  Its
packing is pinned against exact rational results placed chain by chain.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qla_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libqla_oracle.so")
_lib = None

LAYOUTS = {"kv": 0, "vk": 1}
DIRECTIONS = {"fwd": 0, "bwd": 1}


def build(force: bool = False) -> str:
    """Compile ``qla_oracle.c`` into ``libqla_oracle.so`` with gcc (-O2, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH) or (
        os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)
    ):
        tmp = _LIB_PATH + f".tmp{os.getpid()}"
        subprocess.run(
            ["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared",
             "-std=c99", "-Wall", "-Werror", "-o", tmp, _SRC],
            check=True,
        )
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(build())
        fn = lib.qla_oracle_correct_h0
        dp = ctypes.POINTER(ctypes.c_double)
        fn.argtypes = [dp, dp, dp, dp, ctypes.c_int, ctypes.c_int,
                       ctypes.c_long, ctypes.c_int, ctypes.c_int, ctypes.c_int]
        fn.restype = ctypes.c_int
        _lib = lib
    return _lib


def _code(value, table, what):
    if isinstance(value, str):
        if value not in table:
            raise ValueError(f"unknown {what} {value!r}")
        return table[value]
    if int(value) not in table.values():
        raise ValueError(f"unknown {what} {value!r}")
    return int(value)


def _as_f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def correct_h0(H, M, S0, layout, direction):
    """Run the recurrence for every chain of ``H``/``M``; returns fp64 ``out`` shaped like H.

    H: [..., n_seg, K, V] (kv) or [..., n_seg, V, K] (vk); M: [..., n_seg, K, K];
    S0: [..., K, V] / [..., V, K] or None (zero initial state).  Leading dims are
    the chains (batch, heads, ...) and must agree between the arrays.
    """
    lay = _code(layout, LAYOUTS, "layout")
    dire = _code(direction, DIRECTIONS, "direction")
    H = _as_f64(H)
    M = _as_f64(M)
    if H.ndim < 3 or M.ndim != H.ndim:
        raise ValueError("H and M need the same rank >= 3")
    n_seg = H.shape[-3]
    K = M.shape[-1]
    if M.shape[-2] != K or M.shape[:-2] != H.shape[:-2]:
        raise ValueError(f"M shape {M.shape} does not match H shape {H.shape}")
    if lay == 0:
        if H.shape[-2] != K:
            raise ValueError("kv layout needs H[..., K, V]")
        V = H.shape[-1]
    else:
        if H.shape[-1] != K:
            raise ValueError("vk layout needs H[..., V, K]")
        V = H.shape[-2]
    lead = H.shape[:-3]
    chains = int(np.prod(lead)) if lead else 1
    out = np.empty(H.shape, dtype=np.float64)
    dp = ctypes.POINTER(ctypes.c_double)
    s0_ptr = None
    if S0 is not None:
        S0 = _as_f64(S0)
        if S0.shape != lead + H.shape[-2:]:
            raise ValueError(f"S0 shape {S0.shape} does not match H shape {H.shape}")
        s0_ptr = S0.ctypes.data_as(dp)
    rc = _load().qla_oracle_correct_h0(
        H.ctypes.data_as(dp), M.ctypes.data_as(dp), s0_ptr, out.ctypes.data_as(dp),
        lay, dire, chains, n_seg, K, V)
    if rc != 0:
        raise RuntimeError(f"oracle failed with code {rc}")
    return out


def correct_h0_varlen(H, M, S0, seg_offsets, heads, layout, direction):
    """Variable-length chains, by slicing: sequence b has
    n_b = seg_offsets[b+1] - seg_offsets[b] segments, and the packed arrays hold
    the sequences back to back, sequence b's block starting at segment
    heads * seg_offsets[b] and laid out [heads][n_b][K][V] (or [..][V][K] for vk);
    M likewise with K x K; S0 is [n_seqs][heads][..] or None.  Each chain is run
    through ``correct_h0`` (no arithmetic here).  Returns fp64 out shaped like H.

    H and M are given flattened over the segment axis: H [total, R, C] with
    total = heads * seg_offsets[-1]; M [total, K, K].
    """
    offs = [int(x) for x in seg_offsets]
    H = np.asarray(H)
    M = np.asarray(M)
    out = np.zeros(H.shape, dtype=np.float64)
    for b in range(len(offs) - 1):
        n = offs[b + 1] - offs[b]
        for h in range(heads):
            lo = heads * offs[b] + h * n
            if n == 0:
                continue
            s0 = None if S0 is None else np.asarray(S0)[b, h]
            out[lo:lo + n] = correct_h0(H[lo:lo + n], M[lo:lo + n], s0, layout, direction)
    return out
