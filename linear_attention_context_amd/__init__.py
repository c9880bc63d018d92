"""Python binding of libqla.so, the gfx950 context-parallel state-correction library.

Argument marshalling only: every step of the correction runs in the library's
HIP kernels.  The C ABI (include/qla.h) takes device pointers, sizes and a
hipStream_t; these wrappers accept torch tensors (or raw integer addresses),
pass their data pointers and the current HIP stream, and raise on a non-zero
status.  PyTorch is used for device memory and streams only.

There is no fallback: if libqla.so is missing or cannot be loaded, the first
call raises.  Build it with ``python -m linear_attention_context_amd.build``.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "QLA_LAYOUT_KV", "QLA_LAYOUT_VK", "QLA_DIR_FWD", "QLA_DIR_BWD", "QLA_MAX_GROUPS", "QLA_MAX_SEQS",
    "QLA_ERR_MEMORY", "QlaError", "qla_correct_h0", "qla_correct_h0_grouped", "qla_correct_h0_varlen", "qla_status_str",
    "raw_correct_h0", "raw_correct_h0_grouped", "raw_correct_h0_varlen", "load_library", "library_path",
]

QLA_LAYOUT_KV, QLA_LAYOUT_VK = 0, 1
QLA_DIR_FWD, QLA_DIR_BWD = 0, 1
QLA_MAX_GROUPS = 64
QLA_MAX_SEQS = 256
STATUS = {
    0: "QLA_OK", -1: "QLA_ERR_NULL", -2: "QLA_ERR_ENUM", -3: "QLA_ERR_SHAPE", -4: "QLA_ERR_ALIGN",
    -5: "QLA_ERR_ALIAS", -6: "QLA_ERR_GROUPS", -7: "QLA_ERR_LAUNCH", -8: "QLA_ERR_MEMORY",
    -9: "QLA_ERR_SEQS",
}

_PKG = os.path.dirname(os.path.abspath(__file__))
_DEFAULT_LIB = os.path.join(_PKG, "libqla.so")
_libs: dict = {}


class QlaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


class qla_head_group(ctypes.Structure):
    _fields_ = [("head_begin", ctypes.c_int), ("head_count", ctypes.c_int),
                ("layout", ctypes.c_int), ("direction", ctypes.c_int)]


def library_path(variant: str = "") -> str:
    return os.path.join(_PKG, f"libqla{'_' + variant if variant else ''}.so")


def load_library(path: str | None = None) -> ctypes.CDLL:
    """Load (once) and return the library; raises if it is not built."""
    path = path or _DEFAULT_LIB
    lib = _libs.get(path)
    if lib is not None:
        return lib
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is not built; run `python -m linear_attention_context_amd.build` "
            "(there is no fallback path)")
    lib = ctypes.CDLL(path)
    vp, ci = ctypes.c_void_p, ctypes.c_int
    lib.qla_correct_h0.argtypes = [vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, ci, vp]
    lib.qla_correct_h0.restype = ci
    lib.qla_correct_h0_grouped.argtypes = [vp, vp, vp, vp, ctypes.POINTER(qla_head_group), ci,
                                           ci, ci, ci, ci, ci, vp]
    lib.qla_correct_h0_grouped.restype = ci
    lib.qla_correct_h0_varlen.argtypes = [vp, vp, vp, vp, ci, ci, ctypes.POINTER(ci), ci, ci, ci, ci, vp]
    lib.qla_correct_h0_varlen.restype = ci
    lib.qla_status_str.argtypes = [ci]
    lib.qla_status_str.restype = ctypes.c_char_p
    _libs[path] = lib
    return lib


def qla_status_str(status: int, lib: ctypes.CDLL | None = None) -> str:
    return (lib or load_library()).qla_status_str(int(status)).decode()


QLA_ERR_LAUNCH = -7
QLA_ERR_MEMORY = -8
_BAD = object()   # a tensor argument the library must not see
_F32 = None


def _checked_ptr(x, need: int):
    """Pointer of one buffer argument.  A tensor must be float32, contiguous and
    hold at least ``need`` elements (the extent the call reads or writes);
    otherwise ``_BAD``.  Integer addresses and None pass through: the library
    checks those (that a pointer is device memory is always its check)."""
    global _F32
    if x is None:
        return None
    if type(x) is int:
        return x
    if _F32 is None:
        import torch
        _F32 = torch.float32
    try:
        if x.dtype is not _F32 or not x.is_contiguous() or x.numel() < need:
            return _BAD
        return x.data_ptr() or None
    except AttributeError:
        raise TypeError(f"expected a tensor, an int address or None, got {type(x)!r}") from None


def _buffers(H, M, S0, out, states: int, chains: int, K: int, V: int):
    """Pointers of (H, M, S0, out) for ``states`` segment states (K*V floats of
    H and out, K*K of M each) and ``chains`` initial states, or None if a
    tensor is unusable."""
    kv = max(states * K * V, 0)
    ptrs = (_checked_ptr(H, kv), _checked_ptr(M, max(states * K * K, 0)),
            _checked_ptr(S0, max(chains * K * V, 0)), _checked_ptr(out, kv))
    return None if _BAD in ptrs else ptrs


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _enum(value, names):
    if type(value) is int:
        return value
    if isinstance(value, str):
        return names[value]
    return int(value)


_LAYOUT_NAMES = {"kv": QLA_LAYOUT_KV, "vk": QLA_LAYOUT_VK}
_DIR_NAMES = {"fwd": QLA_DIR_FWD, "bwd": QLA_DIR_BWD}


def raw_correct_h0(H, M, S0, out, layout, direction, batch, heads, n_seg, K, V, stream=None,
                   lib: ctypes.CDLL | None = None) -> int:
    """Call qla_correct_h0 and return its status code unchanged (QLA_ERR_MEMORY
    without calling it if a tensor argument is not float32, contiguous, on the
    GPU and large enough)."""
    lib = lib or load_library()
    p = _buffers(H, M, S0, out, batch * heads * n_seg, batch * heads, K, V)
    if p is None:
        return QLA_ERR_MEMORY
    return lib.qla_correct_h0(p[0], p[1], p[2], p[3], _enum(layout, _LAYOUT_NAMES), _enum(direction, _DIR_NAMES),
                              batch, heads, n_seg, K, V, _stream(stream))


def qla_correct_h0(H, M, S0, out, layout, direction, batch, heads, n_seg, K, V, stream=None,
                   lib: ctypes.CDLL | None = None) -> None:
    """Enqueue the correction on ``stream`` (default: torch's current stream); raises QlaError."""
    lib = lib or load_library()
    rc = raw_correct_h0(H, M, S0, out, layout, direction, batch, heads, n_seg, K, V, stream, lib)
    if rc != 0:
        raise QlaError(rc, qla_status_str(rc, lib))


def _groups(groups):
    arr = (qla_head_group * max(len(groups), 1))()
    for i, g in enumerate(groups):
        begin, count, layout, direction = g
        arr[i] = qla_head_group(begin, count, _enum(layout, _LAYOUT_NAMES), _enum(direction, _DIR_NAMES))
    return arr


def raw_correct_h0_grouped(H, M, S0, out, groups, batch, heads, n_seg, K, V, stream=None,
                           lib: ctypes.CDLL | None = None, n_groups: int | None = None) -> int:
    """Call qla_correct_h0_grouped; ``groups`` is a list of (head_begin, head_count, layout, direction)."""
    lib = lib or load_library()
    p = _buffers(H, M, S0, out, batch * heads * n_seg, batch * heads, K, V)
    if p is None:
        return QLA_ERR_MEMORY
    arr = _groups(groups)
    n = len(groups) if n_groups is None else n_groups
    return lib.qla_correct_h0_grouped(p[0], p[1], p[2], p[3], arr, n, batch, heads, n_seg, K, V, _stream(stream))


def qla_correct_h0_grouped(H, M, S0, out, groups, batch, heads, n_seg, K, V, stream=None,
                           lib: ctypes.CDLL | None = None) -> None:
    lib = lib or load_library()
    rc = raw_correct_h0_grouped(H, M, S0, out, groups, batch, heads, n_seg, K, V, stream, lib)
    if rc != 0:
        raise QlaError(rc, qla_status_str(rc, lib))


def raw_correct_h0_varlen(H, M, S0, out, layout, direction, seg_offsets, heads, K, V, stream=None,
                          lib: ctypes.CDLL | None = None, n_seqs: int | None = None) -> int:
    """Call qla_correct_h0_varlen; ``seg_offsets`` is a sequence of n_seqs + 1 ints
    (host memory), or None to pass a NULL pointer."""
    lib = lib or load_library()
    states = chains = 0
    if seg_offsets is None:
        arr, n = None, (0 if n_seqs is None else n_seqs)
    else:
        offs = [int(x) for x in seg_offsets]
        n = len(offs) - 1 if n_seqs is None else n_seqs
        # the library reads n + 1 offsets: never past the array (missing ones read as 0)
        arr = (ctypes.c_int * max(len(offs), n + 1, 1))(*offs)
        if 0 <= n < len(offs):
            states, chains = heads * offs[n], n * heads
    p = _buffers(H, M, S0, out, states, chains, K, V)
    if p is None:
        return QLA_ERR_MEMORY
    return lib.qla_correct_h0_varlen(p[0], p[1], p[2], p[3], _enum(layout, _LAYOUT_NAMES),
                                     _enum(direction, _DIR_NAMES), arr, n, heads, K, V, _stream(stream))


def qla_correct_h0_varlen(H, M, S0, out, layout, direction, seg_offsets, heads, K, V, stream=None,
                          lib: ctypes.CDLL | None = None) -> None:
    """Variable-length chains: sequence b has seg_offsets[b+1] - seg_offsets[b]
    segments; raises QlaError on a non-zero status."""
    lib = lib or load_library()
    rc = raw_correct_h0_varlen(H, M, S0, out, layout, direction, seg_offsets, heads, K, V, stream, lib)
    if rc != 0:
        raise QlaError(rc, qla_status_str(rc, lib))
