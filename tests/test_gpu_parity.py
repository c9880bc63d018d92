"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Tolerance: relative L2 <= 2e-5 per corrected state, and every element within
2e-4 of its state's RMS.  Inputs whose every fp32 product and sum is exact
(signed permutations with small integers; M = 0) must match bit for bit.
"""
import numpy as np
import pytest

import oracle
import qla_inputs as qi
from gpu_util import assert_parity, bits, decode_mismatch, lay, run_hip

pytestmark = pytest.mark.gpu

VARIANTS = [("kv", "fwd"), ("kv", "bwd"), ("vk", "fwd"), ("vk", "bwd")]
# every head dimension the library accepts: K <= 128 runs the producer kernels
# with K/16 MFMA waves, 128 < K < 256 the general kernel zero-padded to 256
ALL_K = list(range(16, 257, 16))


def _ragged_v(K):
    # several 16-column tiles plus a 4-column ragged tail
    return K + 20


@pytest.mark.parametrize("K", ALL_K)
@pytest.mark.parametrize("layout,direction", VARIANTS)
@pytest.mark.parametrize("with_s0", [True, False])
def test_random_small(K, layout, direction, with_s0):
    V = _ragged_v(K)
    H, M, S0 = qi.random_case(100 + K, (2, 3), 5, K, V, with_s0=with_s0)
    ref = oracle.correct_h0(lay(H, layout), M, lay(S0, layout), layout, direction)
    got = run_hip(lay(H, layout), M, lay(S0, layout), layout, direction).cpu().numpy()
    assert_parity(got, ref, f"K={K} V={V} {layout} {direction}")


@pytest.mark.parametrize("K", ALL_K)
@pytest.mark.parametrize("layout,direction", VARIANTS)
def test_signed_permutation_bit_exact(K, layout, direction):
    """Every fp32 product and sum is an exact small integer: GPU == oracle bit for bit."""
    V = _ragged_v(K)
    n = 6
    H = qi.small_integers(7000 + K, (2, 2, n, K, V))
    S0 = qi.small_integers(7002 + K, (2, 2, K, V))
    M = qi.signed_permutations(7001 + K, (2, 2, n), K)
    ref = oracle.correct_h0(lay(H, layout), M, lay(S0, layout), layout, direction)
    got = run_hip(lay(H, layout), M, lay(S0, layout), layout, direction).cpu().numpy()
    want = ref.astype(np.float32)
    assert np.array_equal(ref, want.astype(np.float64)), "reference not exact in fp32"
    assert np.array_equal(bits(got), bits(want)), decode_mismatch(got, want)


@pytest.mark.parametrize("K,V,n", [(64, 64, 12), (128, 128, 8), (256, 256, 16), (128, 84, 5), (16, 16, 5),
                                   (48, 100, 7), (96, 40, 4), (112, 112, 6), (160, 160, 3), (192, 36, 4),
                                   (240, 240, 2)])
@pytest.mark.parametrize("layout,direction", VARIANTS)
def test_coded_sentinel_m_zero(K, V, n, layout, direction):
    """M = 0 and coded H: out must equal H exactly; a mismatch names the segment read."""
    H = qi.coded_states((2, 2), n, K, V)
    M = np.zeros((2, 2, n, K, K), np.float32)
    S0 = np.full((2, 2, K, V), 3.0, np.float32)
    got = run_hip(lay(H, layout), M, lay(S0, layout), layout, direction).cpu().numpy()
    want = lay(H, layout)
    assert np.array_equal(bits(got), bits(want)), decode_mismatch(got, want)


@pytest.mark.parametrize("layout,direction", VARIANTS)
def test_s0_null_equals_zero_buffer(layout, direction):
    H, M, _ = qi.random_case(31, (1, 4), 6, 128, 128, with_s0=False)
    zeros = np.zeros((1, 4, 128, 128), np.float32)
    a = run_hip(lay(H, layout), M, None, layout, direction)
    b = run_hip(lay(H, layout), M, zeros, layout, direction)
    assert np.array_equal(bits(a), bits(b))


@pytest.mark.parametrize("layout,direction", VARIANTS)
def test_in_place_equals_out_of_place(layout, direction):
    H, M, S0 = qi.random_case(32, (2, 2), 7, 128, 100)
    a = run_hip(lay(H, layout), M, lay(S0, layout), layout, direction)
    b = run_hip(lay(H, layout), M, lay(S0, layout), layout, direction, in_place=True)
    assert np.array_equal(bits(a), bits(b))


@pytest.mark.parametrize("n_seg", [1, 2, 3])
def test_short_chains(n_seg):
    """One, two and three segments (odd and even step counts, prologue-only paths)."""
    for layout, direction in VARIANTS:
        H, M, S0 = qi.random_case(40 + n_seg, (1, 5), n_seg, 128, 36)
        ref = oracle.correct_h0(lay(H, layout), M, lay(S0, layout), layout, direction)
        got = run_hip(lay(H, layout), M, lay(S0, layout), layout, direction).cpu().numpy()
        assert_parity(got, ref, f"n_seg={n_seg} {layout} {direction}")


def test_narrow_v_and_chain_counts():
    """V = 4 (one ragged tile) and chain counts that do not fill whole XCD rounds."""
    for V, batch, heads in [(4, 1, 1), (8, 3, 5), (20, 1, 13), (4096, 1, 1)]:
        H, M, S0 = qi.random_case(50 + V, (batch, heads), 3, 64, V)
        for layout, direction in VARIANTS:
            ref = oracle.correct_h0(lay(H, layout), M, lay(S0, layout), layout, direction)
            got = run_hip(lay(H, layout), M, lay(S0, layout), layout, direction).cpu().numpy()
            assert_parity(got, ref, f"V={V} chains={batch}x{heads} {layout} {direction}")


def test_empty_calls_touch_nothing():
    import torch

    import linear_attention_context_amd as qla
    out = torch.full((4, 64, 64), 5.0, device="cuda")
    H = torch.zeros_like(out)
    M = torch.zeros((4, 64, 64), device="cuda")
    for batch, heads, n in [(0, 1, 4), (1, 0, 4), (1, 1, 0)]:
        assert qla.raw_correct_h0(H, M, None, out, "kv", "fwd", batch, heads, n, 64, 64) == 0
    torch.cuda.synchronize()
    assert bool((out == 5.0).all())


@pytest.mark.parametrize("K", [128, 256])
def test_widest_state(K):
    """V = 4096 (256 column tiles) at the larger head dims, both kernels' paths."""
    V = 4096
    H, M, S0 = qi.random_case(70 + K, (1, 1), 2, K, V)
    for layout, direction in VARIANTS:
        ref = oracle.correct_h0(lay(H, layout), M, lay(S0, layout), layout, direction)
        got = run_hip(lay(H, layout), M, lay(S0, layout), layout, direction).cpu().numpy()
        assert_parity(got, ref, f"K={K} V={V} {layout} {direction}")


def test_many_chains():
    """5000 chains of one 16-column tile: a grid far past one workgroup per CU,
    not a multiple of the XCD count, checked on every state."""
    H, M, S0 = qi.random_case(91, (5, 1000), 2, 64, 16)
    for layout, direction in [("kv", "fwd"), ("vk", "bwd")]:
        ref = oracle.correct_h0(lay(H, layout), M, lay(S0, layout), layout, direction)
        got = run_hip(lay(H, layout), M, lay(S0, layout), layout, direction).cpu().numpy()
        assert_parity(got, ref, f"5000 chains {layout} {direction}")


def test_binding_rejects_tensors_the_library_cannot_check():
    """An undersized view of a larger allocation, a bf16 tensor and a transposed
    view all pass the library's allocation-extent check; the binding refuses them."""
    import torch

    import linear_attention_context_amd as qla
    B, NH, N, K, V = 1, 2, 3, 64, 64
    big = torch.zeros(4 * B * NH * N * K * max(K, V), device="cuda")
    need = B * NH * N * K * V
    H = big[:need]
    M = big[need:need + B * NH * N * K * K]
    out = torch.empty(need, device="cuda")
    assert qla.raw_correct_h0(H, M, None, out, "kv", "fwd", B, NH, N, K, V) == 0
    torch.cuda.synchronize()
    assert qla.raw_correct_h0(H[:-1], M, None, out, "kv", "fwd", B, NH, N, K, V) == qla.QLA_ERR_MEMORY
    assert qla.raw_correct_h0(H, M[:-16], None, out, "kv", "fwd", B, NH, N, K, V) == qla.QLA_ERR_MEMORY
    assert qla.raw_correct_h0(H.bfloat16(), M, None, out, "kv", "fwd", B, NH, N, K, V) == qla.QLA_ERR_MEMORY
    Ht = H.view(B * NH * N, K, V).transpose(-1, -2)
    assert qla.raw_correct_h0(Ht, M, None, out, "kv", "fwd", B, NH, N, K, V) == qla.QLA_ERR_MEMORY
    with pytest.raises(qla.QlaError):
        qla.qla_correct_h0(H, M, big[:K * V - 4], out, "kv", "fwd", B, NH, N, K, V)
