"""Host-side checks of the C ABI (no GPU): the library loads, exports every
function include/qla.h declares, and rejects bad arguments before touching the
HIP runtime.  Fake addresses used here are never dereferenced: each call fails
an earlier check (enum, shape, groups, NULL, alignment, overlap)."""
import os
import re
import subprocess

import pytest

import linear_attention_context_amd as qla

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qla.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(qla.library_path()) or not os.path.exists(qla.library_path("delay")):
        from linear_attention_context_amd import build
        build.build()
    return qla.load_library()


def declared_functions():
    text = open(HEADER).read()
    return re.findall(r"QLA_API\s+[\w\s\*]+?\b(qla_\w+)\s*\(", text)


def test_header_declares_four_entry_points():
    assert sorted(declared_functions()) == ["qla_correct_h0", "qla_correct_h0_grouped",
                                            "qla_correct_h0_varlen", "qla_status_str"]


@pytest.mark.parametrize("variant", ["", "delay"])
def test_library_exports_declared_symbols(lib, variant):
    path = qla.library_path(variant)
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    assert set(declared_functions()) <= exported
    # nothing else leaks out of the C ABI
    assert all(name.startswith("qla_") for name in exported), exported


def test_status_strings(lib):
    for code, name in qla.STATUS.items():
        s = qla.qla_status_str(code)
        assert s and s != "unknown status", (code, name)
    assert qla.qla_status_str(12345) == "unknown status"


A = 0x10000000  # fake 16-byte aligned addresses, never dereferenced


def call(**kw):
    args = dict(H=A, M=A + 0x10000000, S0=None, out=A + 0x20000000, layout=0, direction=0,
                batch=1, heads=2, n_seg=3, K=64, V=64, stream=0)
    args.update(kw)
    return qla.raw_correct_h0(**args)


def test_enum_errors(lib):
    assert call(layout=2) == -2
    assert call(direction=-1) == -2


@pytest.mark.parametrize("kw", [dict(K=0), dict(K=8), dict(K=100), dict(K=264), dict(K=272), dict(K=-16),
                                dict(V=6), dict(V=0), dict(V=4100),
                                dict(batch=-1), dict(heads=-2), dict(n_seg=-1),
                                dict(batch=2 ** 30, heads=2 ** 10),
                                # 2^23 workgroups fit an int, but not their work-items a 32-bit count
                                dict(batch=2 ** 23, heads=1, V=16)])
def test_shape_errors(lib, kw):
    assert call(**kw) == -3


def test_size_overflow_rejected(lib):
    """A call whose byte counts would wrap 64 bits is a shape error, not a launch."""
    assert call(batch=2 ** 20, heads=2 ** 10, n_seg=2 ** 30, K=256, V=16) == -3


def test_empty_calls_return_ok_without_pointers(lib):
    for kw in [dict(batch=0), dict(heads=0), dict(n_seg=0)]:
        assert call(H=None, M=None, out=None, **kw) == 0


def test_null_errors(lib):
    assert call(H=None) == -1
    assert call(M=None) == -1
    assert call(out=None) == -1


def test_alignment_errors(lib):
    assert call(H=A + 4) == -4
    assert call(out=A + 0x20000008) == -4
    assert call(S0=A + 0x30000004) == -4


def test_alias_errors(lib):
    state = 64 * 64 * 4
    hbytes = 2 * 3 * state
    # out overlapping H but not identical
    assert call(out=A + 16) == -5
    # out overlapping M
    assert call(out=A + 0x10000000 + 16) == -5
    # out overlapping S0
    assert call(S0=A + 0x20000000 + hbytes - 16) == -5


def groups_call(groups, n_groups=None, heads=4, **kw):
    args = dict(H=A, M=A + 0x10000000, S0=None, out=A + 0x20000000, groups=groups,
                batch=1, heads=heads, n_seg=2, K=64, V=64, stream=0, n_groups=n_groups)
    args.update(kw)
    return qla.raw_correct_h0_grouped(**args)


@pytest.mark.parametrize("groups", [
    [(0, 2, "kv", "fwd"), (1, 3, "vk", "bwd")],        # overlap
    [(0, 1, "kv", "fwd"), (2, 2, "vk", "bwd")],        # gap
    [(0, 2, "kv", "fwd")],                             # does not cover
    [(0, 5, "kv", "fwd")],                             # past heads
    [(-1, 5, "kv", "fwd")],                            # negative begin
    [(0, 0, "kv", "fwd"), (0, 4, "kv", "fwd")],        # empty group
])
def test_group_partition_errors(lib, groups):
    assert groups_call(groups) == -6


def test_group_count_limits(lib):
    assert groups_call([(0, 4, "kv", "fwd")], n_groups=0) == -6
    many = [(i, 1, "kv", "fwd") for i in range(65)]
    assert groups_call(many, heads=65) == -6
    assert groups_call([(0, 4, 3, 0)]) == -2


def test_group_empty_call_ok(lib):
    assert groups_call([(0, 4, "kv", "fwd")], H=None, M=None, out=None, n_seg=0) == 0


def test_binding_raises_with_status(lib):
    with pytest.raises(qla.QlaError) as e:
        qla.qla_correct_h0(A, A + 0x10000000, None, A + 0x20000000, 0, 0, 1, 1, 1, 100, 64, stream=0)
    assert e.value.status == -3


def varlen_call(offs, heads=2, n_seqs=None, **kw):
    args = dict(H=A, M=A + 0x10000000, S0=None, out=A + 0x20000000, layout=0, direction=0,
                seg_offsets=offs, heads=heads, K=64, V=64, stream=0, n_seqs=n_seqs)
    args.update(kw)
    return qla.raw_correct_h0_varlen(**args)


@pytest.mark.parametrize("offs,n_seqs", [
    (None, 2),                 # NULL offsets
    ([1, 3, 5], None),         # first offset not zero
    ([0, 3, 2], None),         # decreasing
    ([0, 3], -1),              # negative count
    ([0] * 258, 257),          # above the sequence limit
])
def test_varlen_offset_errors(lib, offs, n_seqs):
    assert varlen_call(offs, n_seqs=n_seqs) == -9


def test_varlen_enum_and_shape_errors(lib):
    assert varlen_call([0, 2], layout=2) == -2
    assert varlen_call([0, 2], direction=5) == -2
    assert varlen_call([0, 2], K=100) == -3
    assert varlen_call([0, 2], heads=-1) == -3
    assert varlen_call([0, 2 ** 28], heads=16) == -3       # heads * total > INT32_MAX


def test_varlen_empty_calls_ok(lib):
    assert varlen_call([0], H=None, M=None, out=None) == 0              # no sequences
    assert varlen_call([0, 0, 0], H=None, M=None, out=None) == 0        # all empty
    assert varlen_call([0, 4], heads=0, H=None, M=None, out=None) == 0  # no heads


def test_varlen_null_alignment_alias(lib):
    assert varlen_call([0, 2, 5], H=None) == -1
    assert varlen_call([0, 2, 5], out=None) == -1
    assert varlen_call([0, 2, 5], H=A + 4) == -4
    assert varlen_call([0, 2, 5], out=A + 16) == -5


def test_varlen_binding_raises(lib):
    with pytest.raises(qla.QlaError) as e:
        qla.qla_correct_h0_varlen(A, A + 0x10000000, None, A + 0x20000000, 0, 0, [1, 2], 1, 64, 64, stream=0)
    assert e.value.status == -9
