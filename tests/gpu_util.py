"""Helpers for the GPU tests: run the HIP path through the C ABI on numpy inputs
and compare with the fp64 oracle."""
from __future__ import annotations

import numpy as np

import qla_inputs as qi

REL_L2_TOL = 2e-5      # per corrected state, against the fp64 oracle
ELEM_TOL = 2e-4        # per element, relative to the state's RMS (catches localized corruption)


def torch_mod():
    import torch
    return torch


def to_device(a):
    torch = torch_mod()
    if a is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def lay(a, layout):
    """kv-view numpy array -> array stored in ``layout``."""
    if a is None:
        return None
    return a if layout == "kv" else qi.to_vk(a)


def run_hip(H, M, S0, layout, direction, lib=None, in_place=False, out=None):
    """Run qla_correct_h0 on arrays already in ``layout``; returns the device output tensor."""
    import linear_attention_context_amd as qla
    torch = torch_mod()
    b, h, n = H.shape[:3]
    K = M.shape[-1]
    V = H.shape[-1] if layout == "kv" else H.shape[-2]
    Hd, Md, Sd = to_device(H), to_device(M), to_device(S0)
    if in_place:
        out = Hd
    elif out is None:
        out = torch.full_like(Hd, float("nan"))
    print(f"  hip: {layout} {direction} batch={b} heads={h} n_seg={n} K={K} V={V} "
          f"s0={'yes' if S0 is not None else 'no'} in_place={in_place}", flush=True)
    qla.qla_correct_h0(Hd, Md, Sd, out, layout, direction, b, h, n, K, V, lib=lib)
    torch.cuda.synchronize()
    return out


def rel_l2_per_state(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    num = np.sqrt(((got - ref) ** 2).sum(axis=(-1, -2)))
    den = np.sqrt((ref ** 2).sum(axis=(-1, -2)))
    return np.where(den > 0, num / np.where(den > 0, den, 1.0), num)


def assert_parity(got, ref, what=""):
    """Relative L2 per state <= REL_L2_TOL and every element within ELEM_TOL * state RMS."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    rel = rel_l2_per_state(got, ref)
    worst = float(rel.max()) if rel.size else 0.0
    assert worst <= REL_L2_TOL, f"{what}: relative L2 {worst:.3e} > {REL_L2_TOL} at state {np.unravel_index(rel.argmax(), rel.shape)}"
    rms = np.sqrt((ref ** 2).mean(axis=(-1, -2), keepdims=True))
    err = np.abs(got - ref) / np.where(rms > 0, rms, 1.0)
    w = float(err.max()) if err.size else 0.0
    assert w <= ELEM_TOL, f"{what}: element error {w:.3e} x RMS at {np.unravel_index(err.argmax(), err.shape)}"
    return worst


def bits(t):
    """Bit pattern of a float32 tensor/array as int32 numpy."""
    if hasattr(t, "cpu"):
        t = t.cpu().numpy()
    return np.ascontiguousarray(t, np.float32).view(np.int32)


def decode_mismatch(got, want, n_show=5):
    bad = np.argwhere(got != want)
    msgs = []
    for idx in bad[:n_show]:
        idx = tuple(idx)
        g = got[idx]
        msg = f"at {idx}: got {g!r} want {want[idx]!r}"
        if np.isfinite(g) and g >= 1 and float(g).is_integer() and g <= 2 ** 24:
            seg, r, c = qi.decode_code(g)
            msg += f" (value is segment {seg} row {r} col {c}; expected segment {idx[-3]})"
        msgs.append(msg)
    return f"{len(bad)} mismatches; " + "; ".join(msgs)


def oracle_threaded(H, M, S0, layout, direction, threads=None):
    """The fp64 oracle over all chains of (H, M, S0), the chains split across
    host threads (its C loops release the interpreter lock).  Leading axes of H
    and M are the chains; the result is shaped like H."""
    import os
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    lead = H.shape[:-3]
    chains = int(np.prod(lead)) if lead else 1
    Hf = H.reshape((chains,) + H.shape[-3:])
    Mf = M.reshape((chains,) + M.shape[-3:])
    Sf = None if S0 is None else S0.reshape((chains,) + S0.shape[-2:])
    threads = threads or max(1, min(16, len(os.sched_getaffinity(0))))
    bounds = [chains * i // threads for i in range(threads + 1)]
    out = np.empty(Hf.shape, np.float64)

    def part(i):
        lo, hi = bounds[i], bounds[i + 1]
        if hi > lo:
            out[lo:hi] = oracle.correct_h0(Hf[lo:hi], Mf[lo:hi], None if Sf is None else Sf[lo:hi], layout, direction)

    with ThreadPoolExecutor(threads) as pool:
        list(pool.map(part, range(threads)))
    return out.reshape(H.shape)
