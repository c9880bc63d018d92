"""GPU tests of the two-tile producer kernel.

Plain calls at K a multiple of 32 (up to 128) run two tiles of a chain per
workgroup, in two groups of MFMA waves half a step apart, where that saves
rounds of workgroups (tests/test_pair_dispatch.py has the rule).  These shapes
are sized into that range, and each test first checks that the launcher
chooses the two-tile kernel for it.  Every variant is compared with the fp64 oracle: with and without
S0, and with a ragged V whose last pair has one tile only.  Exact inputs and
coded sentinels must come back bit for bit, chains of 1-3 segments exercise
the barrier schedule's ends, and the forced-delay build and repeated calls
must give identical bits.
"""
import ctypes

import numpy as np
import pytest

import oracle
import qla_inputs as qi
from gpu_util import assert_parity, bits, decode_mismatch, lay, oracle_threaded, run_hip, to_device

pytestmark = pytest.mark.gpu

VARIANTS = [("kv", "fwd"), ("kv", "bwd"), ("vk", "fwd"), ("vk", "bwd")]


def _cus():
    import torch
    return torch.cuda.get_device_properties(0).multi_processor_count


def _pair_shape(K, V, n):
    """(batch, heads) for which a plain call runs the two-tile kernel: more
    than three and at most four tiles per compute unit, at most two pair
    workgroups per compute unit."""
    import linear_attention_context_amd as qla
    cus = _cus()
    tiles = (V + 15) // 16
    pairs = (tiles + 1) // 2
    chains = 2 * cus // pairs
    lib = qla.load_library(qla.library_path("delay"))
    lib.qla_test_pairs_tiles.argtypes = [ctypes.c_int, ctypes.c_longlong, ctypes.c_int, ctypes.c_int, ctypes.c_int]
    assert lib.qla_test_pairs_tiles(K, chains, V, n, cus) == 1, (K, chains, V, n, cus)
    return 1, chains


@pytest.mark.parametrize("K", [32, 64, 96, 128])
@pytest.mark.parametrize("layout,direction", VARIANTS)
def test_pair_parity(K, layout, direction):
    V = 100 if K >= 64 else 52  # ragged: 7 or 4 tiles (the last pair of 7 has one tile)
    B, NH = _pair_shape(K, V, 5)
    for with_s0 in (True, False):
        H, M, S0 = qi.random_case(3000 + K, (B, NH), 5, K, V, with_s0=with_s0)
        print(f"  pair K={K} V={V} {B}x{NH} {layout} {direction} s0={with_s0}", flush=True)
        got = run_hip(lay(H, layout), M, lay(S0, layout), layout, direction).cpu().numpy()
        ref = oracle_threaded(lay(H, layout), M, lay(S0, layout), layout, direction)
        assert_parity(got, ref, f"pair K={K} V={V} {B}x{NH} {layout} {direction} s0={with_s0}")


@pytest.mark.parametrize("K", [64, 128])
@pytest.mark.parametrize("layout,direction", VARIANTS)
def test_pair_exact_inputs_and_sentinels(K, layout, direction):
    """Signed permutations with small integers (every fp32 operation exact)
    and the M = 0 coded sentinel: bit for bit."""
    V, n = 128, 4
    B, NH = _pair_shape(K, V, n)
    H = qi.small_integers(3100 + K, (B, NH, n, K, V))
    S0 = qi.small_integers(3102 + K, (B, NH, K, V))
    M = qi.signed_permutations(3101 + K, (B, NH, n), K)
    ref = oracle.correct_h0(lay(H, layout), M, lay(S0, layout), layout, direction)
    want = ref.astype(np.float32)
    assert np.array_equal(ref, want.astype(np.float64))
    got = run_hip(lay(H, layout), M, lay(S0, layout), layout, direction).cpu().numpy()
    assert np.array_equal(bits(got), bits(want)), decode_mismatch(got, want)
    coded = qi.coded_states((B, NH), n, K, V)
    got = run_hip(lay(coded, layout), np.zeros_like(M), lay(S0, layout), layout, direction).cpu().numpy()
    assert np.array_equal(bits(got), bits(lay(coded, layout))), decode_mismatch(got, lay(coded, layout))


@pytest.mark.parametrize("n", [1, 2, 3])
@pytest.mark.parametrize("layout,direction", VARIANTS)
def test_pair_short_chains(n, layout, direction):
    K = V = 128
    B, NH = _pair_shape(K, V, n)
    H, M, S0 = qi.random_case(3200 + n, (B, NH), n, K, V)
    got = run_hip(lay(H, layout), M, lay(S0, layout), layout, direction).cpu().numpy()
    ref = oracle_threaded(lay(H, layout), M, lay(S0, layout), layout, direction)
    assert_parity(got, ref, f"pair n={n} {layout} {direction}")


@pytest.mark.parametrize("layout,direction", VARIANTS)
def test_pair_forced_delay_and_repeat_identical(layout, direction):
    """The forced-delay build gives the same bits; so do 20 repeated calls
    with out cleared to NaN before each."""
    import torch

    import linear_attention_context_amd as qla
    delay = qla.load_library(qla.library_path("delay"))
    K, V, n = 128, 96, 6
    B, NH = _pair_shape(K, V, n)
    H, M, S0 = qi.random_case(3300, (B, NH), n, K, V)
    a = run_hip(lay(H, layout), M, lay(S0, layout), layout, direction)
    b = run_hip(lay(H, layout), M, lay(S0, layout), layout, direction, lib=delay)
    assert np.array_equal(bits(a), bits(b))
    Hd, Md, Sd = to_device(lay(H, layout)), to_device(M), to_device(lay(S0, layout))
    out = torch.empty_like(Hd)
    for _ in range(20):
        out.fill_(float("nan"))
        qla.qla_correct_h0(Hd, Md, Sd, out, layout, direction, B, NH, n, K, V)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32).cpu(), a.view(torch.int32).cpu())


@pytest.mark.parametrize("K", [64, 128])
def test_pair_grouped(K):
    """A grouped call in the two-tile range (the same rule as plain calls):
    every head group against the fp64 oracle, the forced-delay build giving the
    same bits, and a call with one group equal, bit for bit, to the plain call
    of that variant."""
    import torch

    import linear_attention_context_amd as qla
    V, n = 128, 4
    B, NH = _pair_shape(K, V, n)
    q = NH // 4
    groups = [(0, q, "kv", "fwd"), (q, q, "vk", "bwd"), (2 * q, q, "vk", "fwd"), (3 * q, NH - 3 * q, "kv", "bwd")]
    H, M, S0 = qi.random_case(3400 + K, (B, NH), n, K, V)
    # vk heads store V x K matrices; every head is K*V floats per state either way
    Hs, Ss = H.copy(), S0.copy()
    for begin, count, layout, _ in groups:
        if layout == "vk":
            Hs[:, begin:begin + count] = qi.to_vk(H[:, begin:begin + count]).reshape(H[:, begin:begin + count].shape)
            Ss[:, begin:begin + count] = qi.to_vk(S0[:, begin:begin + count]).reshape(S0[:, begin:begin + count].shape)
    Hd, Md, Sd = to_device(Hs), to_device(M), to_device(Ss)
    out = torch.full_like(Hd, float("nan"))
    print(f"  grouped pair K={K} {B}x{NH}", flush=True)
    qla.qla_correct_h0_grouped(Hd, Md, Sd, out, groups, B, NH, n, K, V)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for begin, count, layout, direction in groups:
        sl = slice(begin, begin + count)
        shape = (B, count, n, K, V) if layout == "kv" else (B, count, n, V, K)
        Hh = Hs[:, sl].reshape(shape)
        Sh = Ss[:, sl].reshape(shape[:2] + shape[3:])
        ref = oracle_threaded(Hh, M[:, sl], Sh, layout, direction)
        assert_parity(got[:, sl].reshape(shape), ref, f"grouped pair K={K} {layout} {direction}")
    delayed = torch.full_like(Hd, float("nan"))
    qla.qla_correct_h0_grouped(Hd, Md, Sd, delayed, groups, B, NH, n, K, V,
                               lib=qla.load_library(qla.library_path("delay")))
    torch.cuda.synchronize()
    assert torch.equal(delayed.view(torch.int32), out.view(torch.int32))
    # one group: the plain call's kernel and bits
    one = torch.full_like(Hd, float("nan"))
    qla.qla_correct_h0_grouped(to_device(H), Md, to_device(S0), one, [(0, NH, "kv", "fwd")], B, NH, n, K, V)
    plain = run_hip(H, M, S0, "kv", "fwd")
    torch.cuda.synchronize()
    assert torch.equal(one.view(torch.int32).cpu(), plain.view(torch.int32).cpu())


def _pairs_rule(K, chains, V, n):
    import linear_attention_context_amd as qla
    lib = qla.load_library(qla.library_path("delay"))
    lib.qla_test_pairs_tiles.argtypes = [ctypes.c_int, ctypes.c_longlong, ctypes.c_int, ctypes.c_int, ctypes.c_int]
    return lib.qla_test_pairs_tiles(K, chains, V, n, _cus()) == 1


@pytest.mark.parametrize("layout,direction", VARIANTS)
def test_pair_varlen(layout, direction):
    """Variable-length chains in the two-tile range (judged by the mean chain
    length): ragged lengths with an empty sequence against the fp64 oracle, the
    forced-delay build giving the same bits, and equal lengths bit for bit
    against the fixed-length call."""
    import torch

    import linear_attention_context_amd as qla
    K = V = 128
    heads = 2 * _cus() // 4 // 4  # 4 sequences of `heads` chains: 2 pair workgroups per CU
    seg_counts = [3, 5, 0, 6]
    assert _pairs_rule(K, 4 * heads, V, sum(seg_counts) // 4)
    H, M, S0, offs = qi.varlen_case(3500, seg_counts, heads, K, V)
    ref = oracle.correct_h0_varlen(lay(H, layout), M, lay(S0, layout), offs, heads, layout, direction)
    Hd, Md, Sd = to_device(lay(H, layout)), to_device(M), to_device(lay(S0, layout))
    out = torch.full_like(Hd, float("nan"))
    print(f"  pair varlen {layout} {direction} heads={heads} segs={seg_counts}", flush=True)
    qla.qla_correct_h0_varlen(Hd, Md, Sd, out, layout, direction, offs, heads, K, V)
    torch.cuda.synchronize()
    assert_parity(out.cpu().numpy(), ref, f"pair varlen {layout} {direction}")
    delayed = torch.full_like(Hd, float("nan"))
    qla.qla_correct_h0_varlen(Hd, Md, Sd, delayed, layout, direction, offs, heads, K, V,
                              lib=qla.load_library(qla.library_path("delay")))
    torch.cuda.synchronize()
    assert torch.equal(delayed.view(torch.int32), out.view(torch.int32))
    # equal lengths: the fixed-length call's kernel and bits
    n = 4
    H, M, S0, offs = qi.varlen_case(3600, [n] * 4, heads, K, V)
    Hl, Sl = lay(H, layout), lay(S0, layout)
    Hd, Md, Sd = to_device(Hl), to_device(M), to_device(Sl)
    var = torch.full_like(Hd, float("nan"))
    qla.qla_correct_h0_varlen(Hd, Md, Sd, var, layout, direction, offs, heads, K, V)
    fixed = run_hip(Hl.reshape((4, heads, n) + Hl.shape[1:]), M.reshape(4, heads, n, K, K),
                    Sl.reshape((4, heads) + Sl.shape[2:]), layout, direction)
    torch.cuda.synchronize()
    assert torch.equal(var.view(torch.int32).cpu().flatten(), fixed.view(torch.int32).cpu().flatten())
