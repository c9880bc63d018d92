"""Launch-error reporting on the GPU.

QLA_ERR_LAUNCH is returned when the runtime rejects a launch.  The forced-delay
test library exports qla_test_fail_launches(n), which makes its next n
launches report such a rejection before anything is enqueued; every entry
point must then return QLA_ERR_LAUNCH, leave out untouched, make the binding
raise, and work normally on the next call.  The product library must also not
mistake an error left behind by an unrelated earlier runtime call for a
failure of its own launch.
"""
import ctypes

import pytest

import oracle
import qla_inputs as qi
from gpu_util import assert_parity, to_device

pytestmark = pytest.mark.gpu


def _delay_lib():
    import linear_attention_context_amd as qla
    lib = qla.load_library(qla.library_path("delay"))
    lib.qla_test_fail_launches.argtypes = [ctypes.c_int]
    lib.qla_test_fail_launches.restype = ctypes.c_int
    return lib


def _case():
    H, M, S0 = qi.random_case(4100, (1, 3), 4, 64, 64)
    return H, M, S0


def test_injected_launch_failure_every_entry_point():
    import torch

    import linear_attention_context_amd as qla
    lib = _delay_lib()
    H, M, S0 = _case()
    Hd, Md, Sd = to_device(H), to_device(M), to_device(S0)
    calls = {
        "plain": lambda out: qla.raw_correct_h0(Hd, Md, Sd, out, "kv", "fwd", 1, 3, 4, 64, 64, None, lib),
        "grouped": lambda out: qla.raw_correct_h0_grouped(Hd, Md, Sd, out, [(0, 3, "kv", "fwd")], 1, 3, 4, 64, 64,
                                                          None, lib),
        "varlen": lambda out: qla.raw_correct_h0_varlen(Hd, Md, Sd, out, "kv", "fwd", [0, 4], 3, 64, 64, None, lib),
    }
    ref = oracle.correct_h0(H, M, S0, "kv", "fwd")
    for name, call in calls.items():
        out = torch.full_like(Hd, float("nan"))
        assert lib.qla_test_fail_launches(1) == 0
        assert call(out) == qla.QLA_ERR_LAUNCH, name
        torch.cuda.synchronize()
        assert bool(torch.isnan(out).all()), f"{name}: a rejected launch wrote out"
        assert call(out) == 0, name  # the next call launches
        torch.cuda.synchronize()
        assert_parity(out.cpu().numpy(), ref, f"{name} after a rejected launch")


def test_binding_raises_on_launch_failure():
    import torch

    import linear_attention_context_amd as qla
    lib = _delay_lib()
    H, M, S0 = _case()
    Hd, Md, Sd = to_device(H), to_device(M), to_device(S0)
    out = torch.full_like(Hd, float("nan"))
    assert lib.qla_test_fail_launches(2) == 0
    for _ in range(2):
        with pytest.raises(qla.QlaError) as e:
            qla.qla_correct_h0(Hd, Md, Sd, out, "vk", "bwd", 1, 3, 4, 64, 64, lib=lib)
        assert e.value.status == qla.QLA_ERR_LAUNCH
        assert "QLA_ERR_LAUNCH" in str(e.value)
    qla.qla_correct_h0(Hd, Md, Sd, out, "vk", "bwd", 1, 3, 4, 64, 64, lib=lib)
    torch.cuda.synchronize()
    assert not bool(torch.isnan(out).any())


def test_stale_runtime_error_is_not_a_launch_failure():
    """An unrelated runtime call failed earlier and nobody cleared its error:
    the next correction still launches, returns QLA_OK and is correct."""
    import torch

    import linear_attention_context_amd as qla
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipMalloc.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_size_t]
    hip.hipMalloc.restype = ctypes.c_int
    H, M, S0 = _case()
    Md = to_device(M)
    for layout in ("kv", "vk"):
        Hl = H if layout == "kv" else qi.to_vk(H)
        Sl = S0 if layout == "kv" else qi.to_vk(S0)
        Hd, Sd = to_device(Hl), to_device(Sl)
        out = torch.full_like(Hd, float("nan"))
        p = ctypes.c_void_p()
        assert hip.hipMalloc(ctypes.byref(p), 1 << 60) != 0  # fails: out of memory, error left set
        assert qla.raw_correct_h0(Hd, Md, Sd, out, layout, "fwd", 1, 3, 4, 64, 64) == 0
        torch.cuda.synchronize()
        want = oracle.correct_h0(Hl, M, Sl, layout, "fwd")
        assert_parity(out.cpu().numpy(), want, f"{layout} after a stale runtime error")
