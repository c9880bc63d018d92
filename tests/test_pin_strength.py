"""The pins catch plausible mistakes: each planted mutant fails at least one pin.

Mutants are small numpy implementations of the recurrence with one planted
mistake each.  A correct numpy reference (``_reference``) passes every pin, so
a failure of a mutant is due to its planted mistake, not to the harness.
"""
import numpy as np
import pytest

import pins


def _kvview(a, layout):
    return a if layout == "kv" else np.swapaxes(a, -1, -2)


def _make(mutation=None):
    def impl(H, M, S0, layout, direction):
        H = _kvview(np.asarray(H, np.float64), layout)
        M = np.asarray(M, np.float64)
        n = H.shape[-3]
        lead = H.shape[:-3]
        S = np.zeros(lead + H.shape[-2:]) if S0 is None else \
            _kvview(np.asarray(S0, np.float64), layout).copy()
        if mutation == "vk_s0_untransposed" and layout == "vk" and S0 is not None and S.shape[-1] == S.shape[-2]:
            S = np.asarray(S0, np.float64).copy()
        if mutation == "s0_ignored":
            S = np.zeros_like(S)
        out = np.empty_like(H)
        order = list(range(n)) if direction == "fwd" else list(range(n - 1, -1, -1))
        if mutation == "skip_last" and n > 1:
            order = order[:-1]
        if mutation == "bwd_forward_order" and direction == "bwd":
            order = list(range(n))
        for step, j in enumerate(order):
            Mj = M[..., j, :, :]
            Hj = H[..., j, :, :]
            if mutation == "h_index_shift" and direction == "fwd":
                Hj = H[..., max(j - 1, 0), :, :]
            if mutation == "h_index_shift_bwd" and direction == "bwd":
                Hj = H[..., min(j + 1, n - 1), :, :]
            if mutation == "chain_mix" and H.ndim >= 4 and H.shape[0] > 1:
                Hj = np.roll(H[..., j, :, :], 1, axis=0)
            if mutation == "m_index_shift" and direction == "bwd":
                if j + 1 < n:
                    Mj = M[..., j + 1, :, :]
                else:
                    Mj = np.broadcast_to(np.eye(M.shape[-1]), Mj.shape)
            op = Mj if direction == "fwd" else np.swapaxes(Mj, -1, -2)
            if mutation == "bwd_no_transpose" and direction == "bwd":
                op = Mj
            if mutation == "fwd_transposed" and direction == "fwd":
                op = np.swapaxes(Mj, -1, -2)
            if mutation == "vk_wrong_side" and layout == "vk":
                op = np.swapaxes(op, -1, -2)
            Y = op @ S
            if mutation == "s0_added" and step == 0 and S0 is not None:
                Y = S + Hj * 0.0
            if mutation == "drop_h":
                S_new = Y
            elif mutation == "minus_h":
                S_new = Y - Hj
            else:
                S_new = Y + Hj
            if mutation == "emit_previous":
                out[..., j, :, :] = S
            else:
                out[..., j, :, :] = S_new
            S = S_new
        if mutation == "skip_last" and n > 1:
            out[..., order[-1] + (1 if direction == "fwd" else -1), :, :] = 0.0
        if mutation == "vk_out_untransposed" and layout == "vk" and out.shape[-1] == out.shape[-2]:
            return np.ascontiguousarray(out)
        return np.ascontiguousarray(_kvview(out, layout))
    return impl


MUTATIONS = [
    "drop_h", "minus_h", "bwd_no_transpose", "fwd_transposed", "bwd_forward_order",
    "m_index_shift", "h_index_shift", "s0_ignored", "s0_added", "vk_wrong_side",
    "emit_previous", "vk_s0_untransposed", "vk_out_untransposed", "skip_last", "h_index_shift_bwd",
    "chain_mix",
]


def test_reference_passes_every_pin():
    ref = _make(None)
    for pin in pins.ALL_PINS:
        pin(ref)


@pytest.mark.parametrize("mutation", MUTATIONS)
def test_mutant_fails_a_pin(mutation):
    impl = _make(mutation)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(impl)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin catches mutation {mutation}"
