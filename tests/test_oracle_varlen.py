"""The variable-length oracle: packed ragged chains against the exact rational
result of each chain, placed by the packing that include/qla.h documents
(sequence b's block starts at segment heads * offs[b] and is [heads][n_b][..])."""
import numpy as np
import pytest

import oracle
import pins
import qla_inputs as qi


def _packed_exact(seg_counts, heads, K, V, seed, with_s0, direction):
    rng = qi.rng(seed)
    chains = []
    for n in seg_counts:
        for _ in range(heads):
            H = rng.integers(-8, 9, (n, K, V)) / 4.0
            M = rng.integers(-4, 5, (n, K, K)) / 4.0
            chains.append((H, M))
    S0 = rng.integers(-8, 9, (len(seg_counts), heads, K, V)) / 4.0 if with_s0 else None
    H = np.concatenate([c[0] for c in chains]) if chains else np.zeros((0, K, V))
    M = np.concatenate([c[1] for c in chains]) if chains else np.zeros((0, K, K))
    want = np.zeros_like(H)
    row = 0
    for b, n in enumerate(seg_counts):
        for h in range(heads):
            Hc, Mc = chains[b * heads + h]
            if n:
                ex = pins.unrolled_exact(Hc, Mc, None if S0 is None else S0[b, h], direction)
                want[row:row + n] = np.array([[[float(x) for x in r] for r in s] for s in ex])
            row += n
    offs = np.concatenate([[0], np.cumsum(seg_counts)]).astype(int).tolist()
    return H, M, S0, offs, want


@pytest.mark.parametrize("direction", ["fwd", "bwd"])
@pytest.mark.parametrize("with_s0", [True, False])
def test_varlen_oracle_exact_ragged(direction, with_s0):
    seg_counts, heads, K, V = [2, 0, 3, 1], 2, 2, 3
    H, M, S0, offs, want = _packed_exact(seg_counts, heads, K, V, 31, with_s0, direction)
    got = oracle.correct_h0_varlen(H, M, S0, offs, heads, "kv", direction)
    assert np.array_equal(got, want)
    # the vk layout holds the transposes
    got_vk = oracle.correct_h0_varlen(qi.to_vk(H), M, None if S0 is None else qi.to_vk(S0), offs, heads,
                                      "vk", direction)
    assert np.array_equal(qi.to_vk(got_vk), want)


def test_varlen_oracle_equal_lengths_match_fixed():
    """Equal lengths: the packed layout is [n_seqs][heads][n][..], the fixed-length one."""
    H, M, S0 = qi.random_case(32, (3, 2), 4, 8, 8)
    offs = [0, 4, 8, 12]
    for d in ("fwd", "bwd"):
        fixed = oracle.correct_h0(H, M, S0, "kv", d)
        var = oracle.correct_h0_varlen(H.reshape(-1, 8, 8), M.reshape(-1, 8, 8), S0, offs, 2, "kv", d)
        assert np.array_equal(var.reshape(fixed.shape), fixed)


def test_varlen_inputs_packing():
    H, M, S0, offs = qi.varlen_case(5, [3, 0, 2], 2, 4, 6)
    assert offs == [0, 3, 3, 5]
    assert H.shape == (10, 4, 6) and M.shape == (10, 4, 4) and S0.shape == (3, 2, 4, 6)
    H2, M2, S02 = qi.random_case(7, (2,), 2, 4, 6, 0.9, 0.1, True)
    assert np.array_equal(H[6:], H2.reshape(4, 4, 6)) and np.array_equal(S0[2], S02)
