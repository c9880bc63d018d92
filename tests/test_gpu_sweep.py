"""The pages' operator sweep on the GPU: 4K / 8K / 32K tokens (1, 2, 8 segments of
4096) x 4 / 16 / 32 heads x {kv, vk} x {fwd, bwd} x initial state on / off, at
K = V = 128, batch 1.  Every chain is checked against the fp64 oracle at 4 heads;
at 16 and 32 heads the first, a middle and the last chain are."""
import numpy as np
import pytest

import oracle
import qla_inputs as qi
from gpu_util import assert_parity, lay, run_hip

pytestmark = pytest.mark.gpu

VARIANTS = [("kv", "fwd"), ("vk", "fwd"), ("kv", "bwd"), ("vk", "bwd")]


@pytest.mark.parametrize("tokens", qi.SWEEP_TOKENS)
@pytest.mark.parametrize("heads", qi.SWEEP_HEADS)
def test_sweep_point(tokens, heads):
    H, M, S0 = qi.sweep_arrays(tokens, heads)
    assert H.shape == (1, heads, tokens // qi.SEG_TOKENS, 128, 128)
    chains = range(heads) if heads <= 4 else (0, heads // 2, heads - 1)
    for layout, direction in VARIANTS:
        for s0 in (S0, None):
            got = run_hip(lay(H, layout), M, lay(s0, layout), layout, direction).cpu().numpy()
            assert np.all(np.isfinite(got))
            for h in chains:
                ref = oracle.correct_h0(lay(H, layout)[0, h], M[0, h],
                                        None if s0 is None else lay(s0, layout)[0, h], layout, direction)
                assert_parity(got[0, h], ref, f"{tokens} tokens x {heads} heads, chain {h}, {layout} {direction}, "
                                              f"s0={'on' if s0 is not None else 'off'}")
