"""GPU tests at the five workload sizes, plus determinism and the forced-delay build.

Sizes (batch x heads x segments, K = V):
  1: 1 x 1 x 4, 64, fwd kv           -- oracle on every state
  2: 1 x 32 x 8, 128, fwd kv and vk  -- 32K tokens as 8 segments of 4096; oracle on every state
  3: as 2, bwd kv and vk             -- oracle on every state
  4: 4 x 32 x 64, 128, fwd kv        -- oracle on sampled chains
  5: 2 x 64 x 16, 256, one grouped call, four head groups -- oracle on sampled chains,
     grouped agrees with the per-group plain calls on every chain (parity bar),
     and repeated grouped calls are bit-identical
"""
import numpy as np
import pytest

import oracle
import qla_inputs as qi
from gpu_util import assert_parity, bits, decode_mismatch, lay, run_hip, to_device

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("cfg", [1, 2, 3])
def test_config_full_oracle(cfg):
    case = qi.CASES[cfg]
    H, M, S0 = qi.case_arrays(cfg)
    for layout, direction in case.variants:
        ref = oracle.correct_h0(lay(H, layout), M, lay(S0, layout), layout, direction)
        got = run_hip(lay(H, layout), M, lay(S0, layout), layout, direction).cpu().numpy()
        worst = assert_parity(got, ref, f"config {cfg} {layout} {direction}")
        print(f"  config {cfg} {layout} {direction}: max rel L2 {worst:.3e}", flush=True)


def test_config4_sampled():
    case = qi.CASES[4]
    H, M, S0 = qi.case_arrays(4)
    assert S0 is None
    got = run_hip(H, M, None, "kv", "fwd").cpu().numpy()
    for b, h in [(0, 0), (1, 7), (2, 19), (3, 31)]:
        ref = oracle.correct_h0(H[b, h], M[b, h], None, "kv", "fwd")
        worst = assert_parity(got[b, h], ref, f"config 4 chain ({b},{h})")
        print(f"  config 4 chain ({b},{h}): max rel L2 {worst:.3e}", flush=True)
    assert np.all(np.isfinite(got))
    assert case.n_seg == 64


def _grouped_inputs(H_kv, S0_kv, case):
    """Per-head storage for a grouped call: heads of vk groups hold transposed matrices."""
    H = H_kv.copy()
    S0 = None if S0_kv is None else S0_kv.copy()
    for begin, count, layout, _ in case.group_heads():
        if layout == "vk":
            H[:, begin:begin + count] = qi.to_vk(H_kv[:, begin:begin + count])
            if S0 is not None:
                S0[:, begin:begin + count] = qi.to_vk(S0_kv[:, begin:begin + count])
    return H, S0


def _run_grouped(H, M, S0, case, lib=None):
    import torch

    import linear_attention_context_amd as qla
    Hd, Md, Sd = to_device(H), to_device(M), to_device(S0)
    out = torch.full_like(Hd, float("nan"))
    print(f"  hip grouped: batch={case.batch} heads={case.heads} n_seg={case.n_seg} K={case.K}", flush=True)
    qla.qla_correct_h0_grouped(Hd, Md, Sd, out, case.group_heads(), case.batch, case.heads, case.n_seg,
                               case.K, case.V, lib=lib)
    torch.cuda.synchronize()
    return Hd, Md, Sd, out


def test_config5_grouped():
    case = qi.CASES[5]
    H_kv, M, S0_kv = qi.case_arrays(5)
    H, S0 = _grouped_inputs(H_kv, S0_kv, case)
    Hd, Md, Sd, out = _run_grouped(H, M, S0, case)
    got = out.cpu().numpy()
    # oracle on two chains per group
    for begin, count, layout, direction in case.group_heads():
        for b, h in [(0, begin), (1, begin + count - 1)]:
            ref = oracle.correct_h0(H[b, h], M[b, h], S0[b, h], layout, direction)
            worst = assert_parity(got[b, h], ref, f"config 5 chain ({b},{h}) {layout} {direction}")
            print(f"  config 5 chain ({b},{h}) {layout} {direction}: max rel L2 {worst:.3e}", flush=True)
    # every chain: the grouped launch agrees with the plain entry point on that
    # group's heads.  The two may run a group with different wave counts, and so
    # different fp32 summation orders: agreement is to the parity bar, not bits.
    import torch

    import linear_attention_context_amd as qla
    for b in range(case.batch):
        for begin, count, layout, direction in case.group_heads():
            sl = slice(begin, begin + count)
            sep = torch.full_like(Hd[b, sl], float("nan"))
            qla.qla_correct_h0(Hd[b, sl], Md[b, sl], Sd[b, sl], sep, layout, direction, 1, count,
                               case.n_seg, case.K, case.V)
            torch.cuda.synchronize()
            assert_parity(out[b, sl].cpu().numpy(), sep.cpu().numpy().astype(np.float64),
                          f"grouped vs plain, batch {b} heads {begin}..{begin + count - 1}")


def test_config5_grouped_deterministic():
    """Ten grouped calls at the wide-state size, out cleared to NaN before each: identical bits."""
    import torch

    case = qi.CASES[5]
    H_kv, M, S0_kv = qi.case_arrays(5)
    H, S0 = _grouped_inputs(H_kv, S0_kv, case)
    Hd, Md, Sd, first = _run_grouped(H, M, S0, case)
    first = first.clone()
    import linear_attention_context_amd as qla
    out = torch.empty_like(first)
    for i in range(10):
        out.fill_(float("nan"))
        qla.qla_correct_h0_grouped(Hd, Md, Sd, out, case.group_heads(), case.batch, case.heads, case.n_seg,
                                   case.K, case.V)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), first.view(torch.int32)), f"call {i} differs"


def test_config5_sentinels():
    """Coded H with M = 0 (exact) and the literal segment-id H with config 5's M."""
    case = qi.CASES[5]
    coded = qi.coded_states((case.batch, case.heads), case.n_seg, case.K, case.V)
    M0 = np.zeros((case.batch, case.heads, case.n_seg, case.K, case.K), np.float32)
    S0 = np.full((case.batch, case.heads, case.K, case.V), 1.0, np.float32)
    _, _, _, out = _run_grouped(coded, M0, S0, case)
    got = out.cpu().numpy()
    assert np.array_equal(bits(got), bits(coded)), decode_mismatch(got, coded)
    del got, out, coded, M0

    _, M, S0_kv = qi.case_arrays(5)
    seg_id = np.broadcast_to(np.arange(case.n_seg, dtype=np.float32)[:, None, None],
                             (case.batch, case.heads, case.n_seg, case.K, case.V)).copy()
    H, S0 = _grouped_inputs(seg_id, S0_kv, case)
    _, _, _, out = _run_grouped(H, M, S0, case)
    got = out.cpu().numpy()
    for begin, count, layout, direction in case.group_heads():
        b, h = 1, begin + 3
        ref = oracle.correct_h0(H[b, h], M[b, h], S0[b, h], layout, direction)
        assert_parity(got[b, h], ref, f"literal sentinel ({b},{h}) {layout} {direction}")


@pytest.mark.parametrize("layout,direction", [("kv", "fwd"), ("vk", "fwd"), ("kv", "bwd"), ("vk", "bwd")])
def test_determinism_100_calls(layout, direction):
    """100 calls on the 32K x 32-head shape, out cleared to NaN before each: identical bits."""
    import torch

    import linear_attention_context_amd as qla
    case = qi.CASES[2]
    H, M, S0 = qi.case_arrays(2)
    Hd, Md, Sd = to_device(lay(H, layout)), to_device(M), to_device(lay(S0, layout))
    out = torch.empty_like(Hd)
    first = None
    print(f"  determinism {layout} {direction}: 100 calls", flush=True)
    for i in range(100):
        out.fill_(float("nan"))
        qla.qla_correct_h0(Hd, Md, Sd, out, layout, direction, case.batch, case.heads, case.n_seg,
                           case.K, case.V)
        if first is None:
            torch.cuda.synchronize()
            first = out.clone()
        else:
            assert torch.equal(out.view(torch.int32), first.view(torch.int32)), f"call {i} differs"
    torch.cuda.synchronize()


@pytest.mark.parametrize("layout,direction", [("kv", "fwd"), ("vk", "fwd"), ("kv", "bwd"), ("vk", "bwd")])
def test_forced_delay_build_identical(layout, direction):
    """The library built with one wave per step sleeping before its LDS read and
    before its LDS write produces the same bits (random data and coded sentinel)."""
    import linear_attention_context_amd as qla
    delay = qla.load_library(qla.library_path("delay"))
    H, M, S0 = qi.case_arrays(2)
    a = run_hip(lay(H, layout), M, lay(S0, layout), layout, direction)
    b = run_hip(lay(H, layout), M, lay(S0, layout), layout, direction, lib=delay)
    assert np.array_equal(bits(a), bits(b))
    coded = qi.coded_states((1, 32), 8, 128, 128)
    Mp = qi.signed_permutations(77, (1, 32, 8), 128)
    a = run_hip(lay(coded, layout), Mp, None, layout, direction)
    b = run_hip(lay(coded, layout), Mp, None, layout, direction, lib=delay)
    assert np.array_equal(bits(a), bits(b))
