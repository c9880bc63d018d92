"""GPU tests at the five workload sizes, plus determinism and the forced-delay build.

Sizes (batch x heads x segments, K = V):
  1: 1 x 1 x 4, 64, fwd kv
  2: 1 x 32 x 8, 128, fwd kv and vk  -- 32K tokens as 8 segments of 4096
  3: as 2, bwd kv and vk
  4: 4 x 32 x 64, 128, fwd kv
  5: 2 x 64 x 16, 256, one grouped call, four head groups
Every corrected state of every size is compared with the fp64 oracle (run over
the host's cores).  Repeated calls with out cleared to NaN before each must give
identical bits at every size, and so must the library built with a forced-delay
schedule (one wave per step sleeping before its LDS read and before its LDS
write, one producer copying late), on random and on coded-sentinel inputs.
"""
import numpy as np
import pytest

import oracle
import qla_inputs as qi
from gpu_util import assert_parity, bits, decode_mismatch, lay, oracle_threaded, run_hip, to_device

pytestmark = pytest.mark.gpu

VARIANTS = [("kv", "fwd"), ("vk", "fwd"), ("kv", "bwd"), ("vk", "bwd")]


@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_config_every_state(cfg):
    case = qi.CASES[cfg]
    H, M, S0 = qi.case_arrays(cfg)
    for layout, direction in case.variants:
        got = run_hip(lay(H, layout), M, lay(S0, layout), layout, direction).cpu().numpy()
        ref = oracle_threaded(lay(H, layout), M, lay(S0, layout), layout, direction)
        worst = assert_parity(got, ref, f"config {cfg} {layout} {direction}")
        print(f"  config {cfg} {layout} {direction}: {ref.shape[0] * ref.shape[1]} chains x {case.n_seg} states, "
              f"max rel L2 {worst:.3e}", flush=True)
        del got, ref


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


def _run_grouped(H, M, S0, case, lib=None, out=None):
    import torch

    import linear_attention_context_amd as qla
    Hd, Md, Sd = to_device(H), to_device(M), to_device(S0)
    if out is None:
        out = torch.full_like(Hd, float("nan"))
    print(f"  hip grouped: batch={case.batch} heads={case.heads} n_seg={case.n_seg} K={case.K}", flush=True)
    qla.qla_correct_h0_grouped(Hd, Md, Sd, out, case.group_heads(), case.batch, case.heads, case.n_seg,
                               case.K, case.V, lib=lib)
    torch.cuda.synchronize()
    return Hd, Md, Sd, out


def test_config5_grouped_every_state():
    """The wide mixed call: every chain of every head group against the oracle
    in that group's layout and direction; then, as a second check, each group
    against a plain call on its heads."""
    case = qi.CASES[5]
    H_kv, M, S0_kv = qi.case_arrays(5)
    H, S0 = _grouped_inputs(H_kv, S0_kv, case)
    Hd, Md, Sd, out = _run_grouped(H, M, S0, case)
    got = out.cpu().numpy()
    for begin, count, layout, direction in case.group_heads():
        sl = slice(begin, begin + count)
        ref = oracle_threaded(np.ascontiguousarray(H[:, sl]), np.ascontiguousarray(M[:, sl]),
                              np.ascontiguousarray(S0[:, sl]), layout, direction)
        worst = assert_parity(got[:, sl], ref, f"config 5 heads {begin}..{begin + count - 1} {layout} {direction}")
        print(f"  config 5 {layout} {direction}: {case.batch * count} chains, max rel L2 {worst:.3e}", flush=True)
        del ref
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


def test_config5_sentinels():
    """Coded H with M = 0 (exact) and the literal segment-id H with config 5's M,
    the latter compared with the oracle on every chain."""
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
        sl = slice(begin, begin + count)
        ref = oracle_threaded(np.ascontiguousarray(H[:, sl]), np.ascontiguousarray(M[:, sl]),
                              np.ascontiguousarray(S0[:, sl]), layout, direction)
        assert_parity(got[:, sl], ref, f"literal sentinel heads {begin}.. {layout} {direction}")


def _repeat_identical(launch, out, calls, what):
    import torch
    first = None
    print(f"  determinism {what}: {calls} calls", flush=True)
    for i in range(calls):
        out.fill_(float("nan"))
        launch()
        if first is None:
            torch.cuda.synchronize()
            first = out.clone()
            assert not bool(torch.isnan(first).any()), f"{what}: NaN left in out"
        else:
            assert torch.equal(out.view(torch.int32), first.view(torch.int32)), f"{what}: call {i} differs"
    torch.cuda.synchronize()


@pytest.mark.parametrize("cfg,layout,direction", [(1, "kv", "fwd")] + [(2, lay_, dir_) for lay_, dir_ in VARIANTS]
                         + [(4, "kv", "fwd")])
def test_determinism_100_calls(cfg, layout, direction):
    """100 calls, out cleared to NaN before each: identical bits (configurations
    1, 2/3 in all four variants, and 4)."""
    import torch

    import linear_attention_context_amd as qla
    case = qi.CASES[cfg]
    H, M, S0 = qi.case_arrays(cfg)
    Hd, Md, Sd = to_device(lay(H, layout)), to_device(M), to_device(lay(S0, layout))
    out = torch.empty_like(Hd)
    _repeat_identical(lambda: qla.qla_correct_h0(Hd, Md, Sd, out, layout, direction, case.batch, case.heads,
                                                 case.n_seg, case.K, case.V),
                      out, 100, f"config {cfg} {layout} {direction}")


def test_config5_grouped_determinism_100_calls():
    import torch

    import linear_attention_context_amd as qla
    case = qi.CASES[5]
    H_kv, M, S0_kv = qi.case_arrays(5)
    H, S0 = _grouped_inputs(H_kv, S0_kv, case)
    Hd, Md, Sd = to_device(H), to_device(M), to_device(S0)
    out = torch.empty_like(Hd)
    _repeat_identical(lambda: qla.qla_correct_h0_grouped(Hd, Md, Sd, out, case.group_heads(), case.batch,
                                                         case.heads, case.n_seg, case.K, case.V),
                      out, 100, "config 5 grouped")


def _delay_lib():
    import linear_attention_context_amd as qla
    return qla.load_library(qla.library_path("delay"))


@pytest.mark.parametrize("layout,direction", VARIANTS)
def test_forced_delay_build_identical(layout, direction):
    """32K x 32-head shape (the producer kernel at K = 128): the forced-delay build
    gives the same bits on random data and on coded sentinels with signed
    permutations."""
    delay = _delay_lib()
    H, M, S0 = qi.case_arrays(2)
    a = run_hip(lay(H, layout), M, lay(S0, layout), layout, direction)
    b = run_hip(lay(H, layout), M, lay(S0, layout), layout, direction, lib=delay)
    assert np.array_equal(bits(a), bits(b))
    coded = qi.coded_states((1, 32), 8, 128, 128)
    Mp = qi.signed_permutations(77, (1, 32, 8), 128)
    a = run_hip(lay(coded, layout), Mp, None, layout, direction)
    b = run_hip(lay(coded, layout), Mp, None, layout, direction, lib=delay)
    assert np.array_equal(bits(a), bits(b))


@pytest.mark.parametrize("K", [256, 192, 48])
@pytest.mark.parametrize("layout,direction", VARIANTS)
def test_forced_delay_other_kernels(K, layout, direction):
    """The general kernel (K = 256, and 192 zero-padded to it) and a producer
    kernel with three MFMA waves (K = 48): forced-delay build == normal build,
    bit for bit, on random data (checked against the oracle too) and on
    M = 0 coded sentinels (which must reproduce H exactly)."""
    delay = _delay_lib()
    V, n = (K + 4 if K + 4 <= 256 else K - 4), 7  # a ragged last column tile (coded sentinels need V <= 256)
    H, M, S0 = qi.random_case(1200 + K, (2, 4), n, K, V)
    a = run_hip(lay(H, layout), M, lay(S0, layout), layout, direction)
    b = run_hip(lay(H, layout), M, lay(S0, layout), layout, direction, lib=delay)
    assert np.array_equal(bits(a), bits(b))
    ref = oracle.correct_h0(lay(H, layout), M, lay(S0, layout), layout, direction)
    assert_parity(b.cpu().numpy(), ref, f"delay build K={K} {layout} {direction}")
    coded = qi.coded_states((2, 4), n, K, V)
    M0 = np.zeros((2, 4, n, K, K), np.float32)
    b = run_hip(lay(coded, layout), M0, None, layout, direction, lib=delay).cpu().numpy()
    want = lay(coded, layout)
    assert np.array_equal(bits(b), bits(want)), decode_mismatch(b, want)


@pytest.mark.parametrize("K", [256, 128])
def test_forced_delay_grouped(K):
    """The grouped kernel in the forced-delay build: same bits as the normal
    build, random and coded-sentinel inputs, four head groups."""
    import torch

    import linear_attention_context_amd as qla
    delay = _delay_lib()
    batch, heads, n, V = 2, 8, 6, K
    groups = [(0, 2, "kv", "fwd"), (2, 2, "vk", "fwd"), (4, 2, "kv", "bwd"), (6, 2, "vk", "bwd")]
    H, M, S0 = qi.random_case(1300 + K, (batch, heads), n, K, V)
    coded = qi.coded_states((batch, heads), n, K, V)
    for Hn, Mn in ((H, M), (coded, np.zeros_like(M))):
        Hd, Md, Sd = to_device(Hn), to_device(Mn), to_device(S0)
        outs = []
        for lib in (None, delay):
            out = torch.full_like(Hd, float("nan"))
            qla.qla_correct_h0_grouped(Hd, Md, Sd, out, groups, batch, heads, n, K, V, lib=lib)
            torch.cuda.synchronize()
            outs.append(out)
        assert torch.equal(outs[0].view(torch.int32), outs[1].view(torch.int32)), K
    # the coded run with M = 0 reproduces H exactly in every group
    assert np.array_equal(bits(outs[1]), bits(coded))
