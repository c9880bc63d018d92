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


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        return x.data_ptr() or None
    raise TypeError(f"expected a tensor, an int address or None, got {type(x)!r}")


QLA_ERR_MEMORY = -8


def _tensor_ok(x, need: int) -> bool:
    """A tensor argument must be float32, contiguous, on a GPU and hold at least
    ``need`` elements (the extent the call reads or writes).  Integer
    addresses and None are passed through unchecked: the library checks those."""
    if x is None or isinstance(x, int) or not hasattr(x, "data_ptr"):
        return True
    import torch
    return (x.dtype == torch.float32 and x.is_cuda and x.is_contiguous() and x.numel() >= need)


def _extents_ok(H, M, S0, out, states: int, chains: int, K: int, V: int) -> bool:
    """``states`` segment states of H / out (K*V floats each) and M (K*K), ``chains`` of S0."""
    if states <= 0 or K <= 0 or V <= 0:
        return True  # empty or malformed: the library decides
    return (_tensor_ok(H, states * K * V) and _tensor_ok(out, states * K * V)
            and _tensor_ok(M, states * K * K) and _tensor_ok(S0, chains * K * V))


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _enum(value, names):
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
    if not _extents_ok(H, M, S0, out, batch * heads * n_seg, batch * heads, K, V):
        return QLA_ERR_MEMORY
    return lib.qla_correct_h0(_ptr(H), _ptr(M), _ptr(S0), _ptr(out),
                              _enum(layout, _LAYOUT_NAMES), _enum(direction, _DIR_NAMES),
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
    if not _extents_ok(H, M, S0, out, batch * heads * n_seg, batch * heads, K, V):
        return QLA_ERR_MEMORY
    arr = _groups(groups)
    n = len(groups) if n_groups is None else n_groups
    return lib.qla_correct_h0_grouped(_ptr(H), _ptr(M), _ptr(S0), _ptr(out), arr, n,
                                      batch, heads, n_seg, K, V, _stream(stream))


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
    if seg_offsets is None:
        arr, n = None, (0 if n_seqs is None else n_seqs)
    else:
        offs = [int(x) for x in seg_offsets]
        n = len(offs) - 1 if n_seqs is None else n_seqs
        # the library reads n + 1 offsets: never past the array (missing ones read as 0)
        arr = (ctypes.c_int * max(len(offs), n + 1, 1))(*offs)
        if 0 <= n < len(offs) and not _extents_ok(H, M, S0, out, heads * offs[n], n * heads, K, V):
            return QLA_ERR_MEMORY
    return lib.qla_correct_h0_varlen(_ptr(H), _ptr(M), _ptr(S0), _ptr(out),
                                     _enum(layout, _LAYOUT_NAMES), _enum(direction, _DIR_NAMES),
                                     arr, n, heads, K, V, _stream(stream))


def qla_correct_h0_varlen(H, M, S0, out, layout, direction, seg_offsets, heads, K, V, stream=None,
                          lib: ctypes.CDLL | None = None) -> None:
    """Variable-length chains: sequence b has seg_offsets[b+1] - seg_offsets[b]
    segments; raises QlaError on a non-zero status."""
    lib = lib or load_library()
    rc = raw_correct_h0_varlen(H, M, S0, out, layout, direction, seg_offsets, heads, K, V, stream, lib)
    if rc != 0:
        raise QlaError(rc, qla_status_str(rc, lib))
