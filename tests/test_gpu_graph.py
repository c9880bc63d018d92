"""Graph capture and replay: the library's calls captured in a hipGraph give the
eager result on every replay, with eager work and synchronisation between replays."""
import numpy as np
import pytest

import qla_inputs as qi
from gpu_util import lay, to_device

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager():
    import torch

    import linear_attention_context_amd as qla
    case = qi.CASES[2]
    H, M, S0 = qi.case_arrays(2)
    calls = []
    for layout, direction in [("kv", "fwd"), ("vk", "fwd"), ("kv", "bwd"), ("vk", "bwd")]:
        calls.append(dict(layout=layout, direction=direction, H=to_device(lay(H, layout)), M=to_device(M),
                          S0=to_device(lay(S0, layout))))
    args = (case.batch, case.heads, case.n_seg, case.K, case.V)

    eager = []
    for c in calls:
        out = torch.full_like(c["H"], float("nan"))
        qla.qla_correct_h0(c["H"], c["M"], c["S0"], out, c["layout"], c["direction"], *args)
        eager.append(out)
    torch.cuda.synchronize()

    outs = [torch.full_like(c["H"], float("nan")) for c in calls]
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    print("  capturing 4 calls in a graph", flush=True)
    with torch.cuda.graph(g, stream=cap, capture_error_mode="relaxed"):
        h = torch.cuda.current_stream().cuda_stream
        for c, o in zip(calls, outs):
            qla.qla_correct_h0(c["H"], c["M"], c["S0"], o, c["layout"], c["direction"], *args, stream=h)
    torch.cuda.synchronize()
    for rep in range(4):
        for o in outs:
            o.fill_(float("nan"))  # eager work between replays
        torch.cuda.synchronize()
        print(f"  replay {rep}", flush=True)
        g.replay()
        torch.cuda.synchronize()
        for c, o, e in zip(calls, outs, eager):
            assert torch.equal(o.view(torch.int32), e.view(torch.int32)), (rep, c["layout"], c["direction"])
