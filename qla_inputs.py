"""Seeded synthetic inputs for the CP state-correction recurrence.

This module only draws and arranges input arrays; it holds none of the
recurrence's arithmetic, so both the fp64 oracle (``oracle/``) and the HIP path
(``linear_attention_context_amd``) can be fed from it without sharing code.

Recipe (the same for every consumer):
  * ``numpy.random.Generator(PCG64(seed))`` with ``seed = 1000*cfg + role``,
    role 0 = H, 1 = M, 2 = S0.
  * Standard normal draws in float32, in C order of the kv-view shape
    ``[batch, heads, n_seg, K, V]`` (so chain after chain, segment after segment).
  * ``M = c*I + sqrt(v/K) * Z`` per matrix (``v`` is the variance of the
    perturbation; ``E|Mx|^2 = (c^2 + v)|x|^2 < |x|^2`` keeps long chains bounded).
  * vk-layout inputs are the per-matrix transposes of the same kv-view draws.

The pages measure synthetic operator calls on a 32K-token, 32-head workload;
the head dims, segment count and batch are not printed there, so the shapes
below fix them (K = V = 128, eight 4096-token segments, batch 1 for that case).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

ROLE_H, ROLE_M, ROLE_S0 = 0, 1, 2


@dataclasses.dataclass(frozen=True)
class Case:
    cfg: int
    name: str
    batch: int
    heads: int
    n_seg: int
    K: int
    V: int
    m_diag: float          # c in M = c*I + N(0, v/K)
    m_var: float           # v
    has_s0: bool
    # (layout, direction) per call, or per head group for a grouped call
    variants: tuple
    grouped: bool = False

    @property
    def chains(self) -> int:
        return self.batch * self.heads

    def group_heads(self):
        """Head ranges of a grouped call: equal consecutive groups, one per variant."""
        g = len(self.variants)
        per = self.heads // g
        return [(i * per, per, lay, dire) for i, (lay, dire) in enumerate(self.variants)]


CASES = {
    1: Case(1, "tiny: 1x1 chain, 4 segments, K=V=64, fwd kv", 1, 1, 4, 64, 64,
            0.5, 0.25, False, (("kv", "fwd"),)),
    2: Case(2, "32K tokens x 32 heads: 8 segments of 4096, K=V=128, fwd kv+vk", 1, 32, 8,
            128, 128, 0.9, 0.1, True, (("kv", "fwd"), ("vk", "fwd"))),
    3: Case(3, "32K tokens x 32 heads: 8 segments of 4096, K=V=128, bwd kv+vk", 1, 32, 8,
            128, 128, 0.9, 0.1, True, (("kv", "bwd"), ("vk", "bwd"))),
    4: Case(4, "long chain: 4x32 chains, 64 segments, K=V=128, fwd kv", 4, 32, 64, 128, 128,
            0.95, 0.05, False, (("kv", "fwd"),)),
    5: Case(5, "wide state: 2x64 chains, 16 segments, K=V=256, 4 head groups mixed", 2, 64, 16,
            256, 256, 0.9, 0.1, True,
            (("kv", "fwd"), ("vk", "fwd"), ("kv", "bwd"), ("vk", "bwd")), grouped=True),
}

# Configuration 3 reuses configuration 2's arrays (same shape and distributions).
_SEED_CFG = {1: 1, 2: 2, 3: 2, 4: 4, 5: 5}


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def normal(seed: int, shape) -> np.ndarray:
    return rng(seed).standard_normal(shape, dtype=np.float32)


def propagation_matrices(seed: int, lead: tuple, K: int, diag: float, var: float) -> np.ndarray:
    """``diag*I + N(0, var/K)`` per matrix, float32, shape ``lead + (K, K)``."""
    M = normal(seed, lead + (K, K))
    M *= np.float32(math.sqrt(var / K))
    idx = np.arange(K)
    M[..., idx, idx] += np.float32(diag)
    return M


def to_vk(a: np.ndarray) -> np.ndarray:
    """Per-matrix transpose of a kv-view array (last two axes), as a new C-contiguous array."""
    return np.ascontiguousarray(np.swapaxes(a, -1, -2))


def case_arrays(cfg: int, batch: int | None = None, heads: int | None = None,
                n_seg: int | None = None):
    """kv-view float32 arrays (H, M, S0-or-None) for configuration ``cfg``.

    ``batch``/``heads``/``n_seg`` may shrink the leading dims (a prefix of the
    full draw is NOT taken; a smaller draw with the same seed and recipe is).
    """
    c = CASES[cfg]
    s = _SEED_CFG[cfg]
    b = c.batch if batch is None else batch
    h = c.heads if heads is None else heads
    n = c.n_seg if n_seg is None else n_seg
    H = normal(1000 * s + ROLE_H, (b, h, n, c.K, c.V))
    M = propagation_matrices(1000 * s + ROLE_M, (b, h, n), c.K, c.m_diag, c.m_var)
    S0 = normal(1000 * s + ROLE_S0, (b, h, c.K, c.V)) if c.has_s0 else None
    return H, M, S0


def random_case(seed: int, lead: tuple, n_seg: int, K: int, V: int, diag: float = 0.9,
                var: float = 0.1, with_s0: bool = True):
    """Arbitrary-shape kv-view case with the same recipe (H, S0 ~ N(0,1))."""
    H = normal(1000 * seed + ROLE_H, lead + (n_seg, K, V))
    M = propagation_matrices(1000 * seed + ROLE_M, lead + (n_seg,), K, diag, var)
    S0 = normal(1000 * seed + ROLE_S0, lead + (K, V)) if with_s0 else None
    return H, M, S0


def signed_permutations(seed: int, lead: tuple, K: int) -> np.ndarray:
    """One random signed permutation matrix per index of ``lead``: M[a, perm[a]] = +-1."""
    g = rng(seed)
    count = int(np.prod(lead)) if lead else 1
    M = np.zeros((count, K, K), dtype=np.float32)
    for i in range(count):
        perm = g.permutation(K)
        sign = g.choice(np.array([-1.0, 1.0], dtype=np.float32), size=K)
        M[i, np.arange(K), perm] = sign
    return M.reshape(lead + (K, K))


def small_integers(seed: int, shape, lo: int = -8, hi: int = 8) -> np.ndarray:
    """Uniform integers in [lo, hi] as float32 (exact in every fp32 sum used here)."""
    return rng(seed).integers(lo, hi + 1, size=shape).astype(np.float32)


def coded_states(lead: tuple, n_seg: int, R: int, C: int) -> np.ndarray:
    """Sentinel H: element (j, r, c) holds j*2^16 + r*2^8 + c + 1 (exact in fp32).

    Needs n_seg <= 256 and R, C <= 256; the value decodes back to (segment, row,
    column), so a read of another segment's data names the segment it came from.
    """
    if n_seg > 256 or R > 256 or C > 256:
        raise ValueError("coded sentinel needs n_seg, R, C <= 256")
    j = np.arange(n_seg, dtype=np.int64)[:, None, None]
    r = np.arange(R, dtype=np.int64)[None, :, None]
    c = np.arange(C, dtype=np.int64)[None, None, :]
    code = (j << 16) + (r << 8) + c + 1
    return np.broadcast_to(code.astype(np.float32), lead + (n_seg, R, C)).copy()


def decode_code(value) -> tuple:
    x = int(value) - 1
    return x >> 16, (x >> 8) & 255, x & 255


# The pages' operator sweep (correction note, section "性能结果"): sequence
# lengths 4K / 8K / 32K tokens and 4 / 16 / 32 heads, both layouts and
# directions, with and without an initial state, at K = V = 128.  Segments
# are 4096 tokens, so the lengths are 1, 2 and 8 segments; batch 1.
SEG_TOKENS = 4096
SWEEP_TOKENS = (4096, 8192, 32768)
SWEEP_HEADS = (4, 16, 32)


def sweep_arrays(tokens: int, heads: int):
    """kv-view (H, M, S0) for one sweep point: the 32K x 32-head recipe
    (M = 0.9 I + N(0, 0.1/K), H and S0 ~ N(0, 1)) at its own seed."""
    ti, hi = SWEEP_TOKENS.index(tokens), SWEEP_HEADS.index(heads)
    return random_case(60 + 3 * ti + hi, (1, heads), tokens // SEG_TOKENS, 128, 128, 0.9, 0.1, True)



def varlen_case(seed: int, seg_counts, heads: int, K: int, V: int, with_s0: bool = True):
    """Packed kv-view inputs for variable-length chains: sequence b (with
    seg_counts[b] segments) is drawn as ``random_case(seed + b, (heads,), n_b,
    K, V)`` and the sequences are stored back to back along the segment axis.
    Returns (H [total, K, V], M [total, K, K], S0 [n_seqs, heads, K, V] or None,
    seg_offsets) with total = heads * sum(seg_counts)."""
    offs = [0]
    for n in seg_counts:
        offs.append(offs[-1] + int(n))
    Hs, Ms, S0s = [], [], []
    for b, n in enumerate(seg_counts):
        H, M, S0 = random_case(seed + b, (heads,), int(n), K, V, 0.9, 0.1, with_s0)
        Hs.append(H.reshape(heads * int(n), K, V))
        Ms.append(M.reshape(heads * int(n), K, K))
        if with_s0:
            S0s.append(S0)
    H = np.concatenate(Hs, axis=0) if Hs else np.zeros((0, K, V), np.float32)
    M = np.concatenate(Ms, axis=0) if Ms else np.zeros((0, K, K), np.float32)
    S0 = np.stack(S0s, axis=0) if with_s0 and S0s else None
    return H, M, S0, offs
