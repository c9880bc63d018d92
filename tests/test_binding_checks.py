"""The binding refuses tensors the library cannot check itself (CPU only).

The C ABI sees raw pointers; under PyTorch's caching allocator the runtime's
allocation extent is a whole cached segment, not the tensor, so a too-small
view, a wrong dtype or a strided view would pass the library's own checks.
The binding therefore checks every tensor argument first and returns
QLA_ERR_MEMORY (-8) without calling the library.  (Whether a pointer is
device memory at all stays the library's check.)
"""
import pytest
import torch

import linear_attention_context_amd as qla


class FakeTensor:
    """Stands in for a device tensor: only what the binding's checks read."""

    def __init__(self, numel, dtype=torch.float32, contiguous=True, ptr=0x10000000):
        self._n, self.dtype, self._c, self._p = numel, dtype, contiguous, ptr

    def numel(self):
        return self._n

    def is_contiguous(self):
        return self._c

    def data_ptr(self):
        return self._p


class NoLib:
    """A library handle that fails the test if the binding calls an entry point."""

    @staticmethod
    def qla_status_str(code):
        return b"a buffer is not device memory or is smaller than the call needs"

    def __getattr__(self, name):
        raise AssertionError(f"the binding called {name} for a rejected tensor")


B, NH, N, K, V = 2, 3, 4, 32, 20
STATES = B * NH * N


def args(**kw):
    a = dict(H=FakeTensor(STATES * K * V), M=FakeTensor(STATES * K * K), S0=FakeTensor(B * NH * K * V),
             out=FakeTensor(STATES * K * V, ptr=0x20000000))
    a.update(kw)
    return a


@pytest.mark.parametrize("bad", [
    dict(H=FakeTensor(STATES * K * V - 1)),                       # one element short
    dict(out=FakeTensor(STATES * K * V - 4, ptr=0x20000000)),
    dict(M=FakeTensor(STATES * K * K - 1)),
    dict(S0=FakeTensor(B * NH * K * V - 1)),
    dict(H=FakeTensor(STATES * K * V, dtype=torch.bfloat16)),     # wrong dtype
    dict(M=FakeTensor(STATES * K * K, dtype=torch.float64)),
    dict(out=FakeTensor(STATES * K * V, contiguous=False)),       # a strided view
])
def test_rejected_before_the_library(bad):
    a = args(**bad)
    rc = qla.raw_correct_h0(a["H"], a["M"], a["S0"], a["out"], "kv", "fwd", B, NH, N, K, V, stream=0, lib=NoLib())
    assert rc == qla.QLA_ERR_MEMORY
    rc = qla.raw_correct_h0_grouped(a["H"], a["M"], a["S0"], a["out"], [(0, NH, "kv", "fwd")], B, NH, N, K, V,
                                    stream=0, lib=NoLib())
    assert rc == qla.QLA_ERR_MEMORY
    # variable-length: two sequences of N segments each is the same extent
    rc = qla.raw_correct_h0_varlen(a["H"], a["M"], a["S0"], a["out"], "kv", "fwd", [0, N, 2 * N], NH, K, V,
                                   stream=0, lib=NoLib())
    assert rc == qla.QLA_ERR_MEMORY


def test_raising_wrapper_names_the_status():
    a = args(H=FakeTensor(10))
    with pytest.raises(qla.QlaError) as e:
        qla.qla_correct_h0(a["H"], a["M"], a["S0"], a["out"], "kv", "fwd", B, NH, N, K, V, stream=0, lib=NoLib())
    assert e.value.status == qla.QLA_ERR_MEMORY


def test_exact_extents_and_addresses_pass_through():
    """Exactly large enough tensors, integer addresses and a NULL S0 reach the library."""
    calls = []

    class Rec:
        def qla_correct_h0(self, *a):
            calls.append(a)
            return 0

    a = args()
    assert qla.raw_correct_h0(a["H"], a["M"], None, a["out"], "kv", "fwd", B, NH, N, K, V, stream=0, lib=Rec()) == 0
    assert qla.raw_correct_h0(0x10000000, 0x30000000, None, 0x20000000, "kv", "fwd", B, NH, N, K, V, stream=0,
                              lib=Rec()) == 0
    assert len(calls) == 2
