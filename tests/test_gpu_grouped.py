"""GPU parity of qla_correct_h0_grouped at every head dim: uneven head groups
(layout and direction chosen per group), a ragged V tail, with and without S0,
against the fp64 oracle on every chain."""
import numpy as np
import pytest

import oracle
import qla_inputs as qi
from gpu_util import assert_parity, to_device

pytestmark = pytest.mark.gpu

GROUPS = [(0, 1, "vk", "bwd"), (1, 2, "kv", "fwd"), (3, 3, "vk", "fwd"), (6, 1, "kv", "bwd")]


@pytest.mark.parametrize("K", [16, 48, 64, 96, 128, 160, 224, 256])
@pytest.mark.parametrize("with_s0", [True, False])
def test_grouped_uneven(K, with_s0):
    import torch

    import linear_attention_context_amd as qla
    batch, heads, n, V = 2, 7, 3, K + 20
    H_kv, M, S0_kv = qi.random_case(500 + K, (batch, heads), n, K, V, with_s0=with_s0)
    # vk heads store V x K matrices: build each head's storage, then pack them
    per_head = []
    for h in range(heads):
        layout = next(l for b, c, l, _ in GROUPS if b <= h < b + c)
        per_head.append(qi.to_vk(H_kv[:, h]) if layout == "vk" else H_kv[:, h])
    print(f"  grouped K={K} V={V} s0={with_s0}", flush=True)
    # every head is K*V floats per state whatever its layout: pack them flat
    flat = np.stack([p.reshape(batch, n, K * V) for p in per_head], axis=1)
    s0_flat = None
    if S0_kv is not None:
        s0_heads = []
        for h in range(heads):
            layout = next(l for b, c, l, _ in GROUPS if b <= h < b + c)
            s0_heads.append((qi.to_vk(S0_kv[:, h]) if layout == "vk" else S0_kv[:, h]).reshape(batch, K * V))
        s0_flat = np.stack(s0_heads, axis=1)
    Hd, Md, Sd = to_device(flat), to_device(M), to_device(s0_flat)
    out = torch.full_like(Hd, float("nan"))
    qla.qla_correct_h0_grouped(Hd, Md, Sd, out, GROUPS, batch, heads, n, K, V)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for begin, count, layout, direction in GROUPS:
        for h in range(begin, begin + count):
            shape = (batch, n, K, V) if layout == "kv" else (batch, n, V, K)
            Hh = flat[:, h].reshape(shape)
            Sh = None if s0_flat is None else s0_flat[:, h].reshape(shape[:1] + shape[2:])
            ref = oracle.correct_h0(Hh, M[:, h], Sh, layout, direction)
            assert_parity(got[:, h].reshape(shape), ref, f"K={K} head {h} {layout} {direction}")


def test_grouped_in_place():
    """out == H for a grouped call: the same bits as a separate out buffer."""
    import torch

    import linear_attention_context_amd as qla
    batch, heads, n, K = 1, 7, 4, 128
    H_kv, M, S0_kv = qi.random_case(777, (batch, heads), n, K, K)
    Hd, Md, Sd = to_device(H_kv), to_device(M), to_device(S0_kv)
    sep = torch.full_like(Hd, float("nan"))
    qla.qla_correct_h0_grouped(Hd, Md, Sd, sep, GROUPS, batch, heads, n, K, K)
    torch.cuda.synchronize()
    qla.qla_correct_h0_grouped(Hd, Md, Sd, Hd, GROUPS, batch, heads, n, K, K)
    torch.cuda.synchronize()
    assert torch.equal(Hd.view(torch.int32), sep.view(torch.int32))


@pytest.mark.parametrize("K", [32, 64, 112, 128, 160, 256])
def test_grouped_matches_plain_calls_bitwise(K):
    """A grouped call runs the same per-chain code as plain calls (at K > 128 as
    one launch per direction, with the plain kernels' block shapes): every
    group's output equals, bit for bit, a plain call on that group's heads."""
    import torch

    import linear_attention_context_amd as qla
    batch, heads, n, V = 2, 7, 5, K + 20
    H, M, S0 = qi.random_case(900 + K, (batch, heads), n, K, V)
    # all heads stored in the kv shape; vk groups read their heads' K*V floats as V x K
    Hd, Md, Sd = to_device(H), to_device(M), to_device(S0)
    grouped = torch.full_like(Hd, float("nan"))
    qla.qla_correct_h0_grouped(Hd, Md, Sd, grouped, GROUPS, batch, heads, n, K, V)
    torch.cuda.synchronize()
    for begin, count, layout, direction in GROUPS:
        sl = slice(begin, begin + count)
        h = to_device(np.ascontiguousarray(H[:, sl]))
        m = to_device(np.ascontiguousarray(M[:, sl]))
        s = to_device(np.ascontiguousarray(S0[:, sl]))
        plain = torch.full_like(h, float("nan"))
        if layout == "vk":  # the same floats, viewed V x K
            h, s, plain = h.view(batch, count, n, V, K), s.view(batch, count, V, K), plain.view(batch, count, n, V, K)
        qla.qla_correct_h0(h, m, s, plain, layout, direction, batch, count, n, K, V)
        torch.cuda.synchronize()
        g = grouped[:, sl].contiguous().view(torch.int32).flatten()
        assert torch.equal(g, plain.contiguous().view(torch.int32).flatten()), (K, begin, layout, direction)
