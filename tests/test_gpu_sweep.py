"""The pages' operator sweep on the GPU: 4K / 8K / 32K tokens (1, 2, 8 segments of
4096) x 4 / 16 / 32 heads x {kv, vk} x {fwd, bwd} x initial state on / off, at
K = V = 128, batch 1.  Every chain of every point is checked against the fp64
oracle (run over the host's cores)."""
import pytest

import qla_inputs as qi
from gpu_util import assert_parity, lay, oracle_threaded, run_hip

pytestmark = pytest.mark.gpu

VARIANTS = [("kv", "fwd"), ("vk", "fwd"), ("kv", "bwd"), ("vk", "bwd")]


@pytest.mark.parametrize("tokens", qi.SWEEP_TOKENS)
@pytest.mark.parametrize("heads", qi.SWEEP_HEADS)
def test_sweep_point(tokens, heads):
    H, M, S0 = qi.sweep_arrays(tokens, heads)
    assert H.shape == (1, heads, tokens // qi.SEG_TOKENS, 128, 128)
    for layout, direction in VARIANTS:
        for s0 in (S0, None):
            got = run_hip(lay(H, layout), M, lay(s0, layout), layout, direction).cpu().numpy()
            ref = oracle_threaded(lay(H, layout), M, lay(s0, layout), layout, direction)
            assert_parity(got, ref, f"{tokens} tokens x {heads} heads, {layout} {direction}, "
                                    f"s0={'on' if s0 is not None else 'off'}")
