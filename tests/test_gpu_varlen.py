"""GPU parity of qla_correct_h0_varlen: ragged chains (including empty ones) in
the packed layout, every variant, K = 48 / 64 / 96 / 128 / 192 / 256, with and without S0,
against the fp64 oracle on every state; equal lengths give the bits of the
fixed-length entry point; in place; the all-empty call writes nothing."""
import numpy as np
import pytest

import oracle
import qla_inputs as qi
from gpu_util import assert_parity, bits, lay, to_device

pytestmark = pytest.mark.gpu

VARIANTS = [("kv", "fwd"), ("vk", "fwd"), ("kv", "bwd"), ("vk", "bwd")]


def run_varlen(H, M, S0, offs, heads, layout, direction, K, V, in_place=False):
    import torch

    import linear_attention_context_amd as qla
    Hd, Md, Sd = to_device(H), to_device(M), to_device(S0)
    out = Hd if in_place else torch.full_like(Hd, float("nan"))
    print(f"  hip varlen: {layout} {direction} offs={offs} heads={heads} K={K} V={V} "
          f"s0={'yes' if S0 is not None else 'no'} in_place={in_place}", flush=True)
    qla.qla_correct_h0_varlen(Hd, Md, Sd, out, layout, direction, offs, heads, K, V)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("K,V,heads,seg_counts", [
    (64, 64, 4, [5, 0, 1, 9, 3]),
    (128, 128, 3, [0, 7, 2, 12]),
    (128, 80, 2, [4, 1, 0, 0, 6]),     # ragged V tail: 16-column tiles over 80
    (256, 256, 2, [3, 0, 6]),
    (48, 52, 3, [2, 5, 0, 1]),         # K = 48: three MFMA waves, uneven producer shares
    (96, 96, 2, [3, 0, 4]),
    (192, 100, 2, [2, 5]),             # zero-padded to the K = 256 kernel
])
@pytest.mark.parametrize("with_s0", [True, False])
def test_varlen_parity(K, V, heads, seg_counts, with_s0):
    H, M, S0, offs = qi.varlen_case(300 + K + len(seg_counts), seg_counts, heads, K, V, with_s0)
    for layout, direction in VARIANTS:
        ref = oracle.correct_h0_varlen(lay(H, layout), M, lay(S0, layout), offs, heads, layout, direction)
        got = run_varlen(lay(H, layout), M, lay(S0, layout), offs, heads, layout, direction, K, V)
        worst = assert_parity(got, ref, f"varlen K={K} V={V} {layout} {direction}")
        print(f"    max rel L2 {worst:.3e}", flush=True)


@pytest.mark.parametrize("layout,direction", VARIANTS)
def test_varlen_equal_lengths_bit_identical_to_fixed(layout, direction):
    """Equal lengths: the packing is the fixed-length [batch][heads][n] layout and
    the same kernel code runs, so the bits agree."""
    import torch

    import linear_attention_context_amd as qla
    case = qi.CASES[2]
    H, M, S0 = qi.case_arrays(2)
    Hl, Sl = lay(H, layout), lay(S0, layout)
    Hd, Md, Sd = to_device(Hl), to_device(M), to_device(Sl)
    fixed = torch.full_like(Hd, float("nan"))
    qla.qla_correct_h0(Hd, Md, Sd, fixed, layout, direction, case.batch, case.heads, case.n_seg, case.K, case.V)
    var = torch.full_like(Hd, float("nan"))
    offs = [b * case.n_seg for b in range(case.batch + 1)]
    qla.qla_correct_h0_varlen(Hd, Md, Sd, var, layout, direction, offs, case.heads, case.K, case.V)
    torch.cuda.synchronize()
    assert np.array_equal(bits(fixed), bits(var))


@pytest.mark.parametrize("layout,direction", VARIANTS)
def test_varlen_in_place(layout, direction):
    seg_counts, heads, K, V = [6, 0, 3], 2, 128, 128
    H, M, S0, offs = qi.varlen_case(411, seg_counts, heads, K, V, True)
    ref = oracle.correct_h0_varlen(lay(H, layout), M, lay(S0, layout), offs, heads, layout, direction)
    got = run_varlen(lay(H, layout), M, lay(S0, layout), offs, heads, layout, direction, K, V, in_place=True)
    assert_parity(got, ref, f"varlen in place {layout} {direction}")


def test_varlen_all_empty_writes_nothing():
    import torch

    import linear_attention_context_amd as qla
    Hd = torch.ones(4, 64, 64, device="cuda")
    Md = torch.ones(4, 64, 64, device="cuda")
    out = torch.full_like(Hd, 7.0)
    qla.qla_correct_h0_varlen(Hd, Md, None, out, "kv", "fwd", [0, 0, 0], 2, 64, 64)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())


def test_varlen_host_pointer_rejected():
    """H in pageable host memory is rejected before any launch."""
    import torch

    import linear_attention_context_amd as qla
    host = np.zeros((4, 64, 64), np.float32)
    Md = torch.zeros(4, 64, 64, device="cuda")
    out = torch.zeros(4, 64, 64, device="cuda")
    rc = qla.raw_correct_h0_varlen(host.ctypes.data, Md, None, out, "kv", "fwd", [0, 1, 2], 2, 64, 64)
    assert rc == -8
    torch.cuda.synchronize()


def test_varlen_deterministic():
    """Ten calls with out cleared to NaN before each: identical bits."""
    import torch

    import linear_attention_context_amd as qla
    H, M, S0, offs = qi.varlen_case(421, [3, 0, 5, 1], 4, 128, 128, True)
    Hd, Md, Sd = to_device(H), to_device(M), to_device(S0)
    out = torch.empty_like(Hd)
    first = None
    for i in range(10):
        out.fill_(float("nan"))
        qla.qla_correct_h0_varlen(Hd, Md, Sd, out, "kv", "fwd", offs, 4, 128, 128)
        torch.cuda.synchronize()
        if first is None:
            first = out.clone()
        else:
            assert torch.equal(out.view(torch.int32), first.view(torch.int32)), f"call {i} differs"
