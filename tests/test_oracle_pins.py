"""The fp64 oracle against its pins (closed forms, exact brute force, invariants, golden)."""
import numpy as np
import pytest

import oracle
import pins


def _oracle(H, M, S0, layout, direction):
    return oracle.correct_h0(H, M, S0, layout, direction)


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(_oracle)


def test_oracle_layout_transpose_bit_identical():
    """kv and vk branches run the same products in the same order: identical bits."""
    import qla_inputs as qi
    H, M, S0 = qi.random_case(21, (3,), 5, 16, 24)
    for d in ("fwd", "bwd"):
        kv = oracle.correct_h0(H, M, S0, "kv", d)
        vk = oracle.correct_h0(qi.to_vk(H), M, qi.to_vk(S0), "vk", d)
        assert np.array_equal(qi.to_vk(vk), kv)


def test_oracle_reverse_bit_identical():
    import qla_inputs as qi
    H, M, S0 = qi.random_case(22, (2,), 6, 8, 8)
    Mt_rev = np.ascontiguousarray(np.swapaxes(M, -1, -2)[:, ::-1])
    bwd = oracle.correct_h0(H, M, S0, "kv", "bwd")
    fwd = oracle.correct_h0(np.ascontiguousarray(H[:, ::-1]), Mt_rev, S0, "kv", "fwd")
    assert np.array_equal(bwd, fwd[:, ::-1])


def test_oracle_empty_and_shapes():
    H = np.zeros((2, 0, 4, 4), np.float32)
    M = np.zeros((2, 0, 4, 4), np.float32)
    assert oracle.correct_h0(H, M, None, "kv", "fwd").shape == (2, 0, 4, 4)
    with pytest.raises(ValueError):
        oracle.correct_h0(np.zeros((1, 2, 4, 5)), np.zeros((1, 2, 4, 4)), None, "vk", "fwd")
    with pytest.raises(ValueError):
        oracle.correct_h0(np.zeros((1, 2, 4, 5)), np.zeros((1, 2, 4, 4)), None, "kv", "up")


def test_oracle_chains_independent():
    """A chain's result does not depend on the other chains in the call."""
    import qla_inputs as qi
    H, M, S0 = qi.random_case(23, (2, 3), 4, 8, 8)
    full = oracle.correct_h0(H, M, S0, "kv", "bwd")
    one = oracle.correct_h0(H[1, 2], M[1, 2], S0[1, 2], "kv", "bwd")
    assert np.array_equal(full[1, 2], one)
