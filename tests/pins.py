"""Pins for the CP state-correction recurrence: checks that do not trust the oracle.

Each ``pin_*`` takes an implementation ``impl(H, M, S0, layout, direction) -> out``
(numpy in, fp64 numpy out) and raises ``AssertionError`` when the implementation
disagrees with something fixed independently of it: a closed form, an exact
rational brute force, an invariant of the linear map, or a hand-worked example.
The oracle must pass all of them; ``test_pin_strength.py`` shows that planted
mistakes (dropped term, wrong sign, wrong transpose, shifted index, wrong
order, wrong side) each fail at least one.

The recurrence (Antarx Memos, FlashQLA correction note, sections "从版本升级后的
数值偏差开始" and "理解三个缓冲区，才能判断哪里需要同步"): forward
S_j = M_j S_{j-1} + H_j for j ascending; backward G_j = M_j^T G_{j+1} + H_j for
j descending; kv stores the K x V state, vk its transpose; S0 (or zero) starts
the chain.
"""
from __future__ import annotations

import json
import os
from fractions import Fraction

import numpy as np

import qla_inputs as qi

LAYOUTS = ("kv", "vk")
DIRECTIONS = ("fwd", "bwd")
GOLDEN_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _lay(a, layout):
    """kv-view array -> array in the given layout (vk = per-matrix transpose)."""
    return a if layout == "kv" else qi.to_vk(a)


def _kv(a, layout):
    return a if layout == "kv" else qi.to_vk(a)


# ---------------------------------------------------------------- closed forms
def pin_m_zero(impl, seed=11):
    """M = 0: every corrected state equals its local state, for any S0 (exact)."""
    H, _, S0 = qi.random_case(seed, (2,), 5, 8, 12)
    M = np.zeros((2, 5, 8, 8), np.float32)
    for lay in LAYOUTS:
        for d in DIRECTIONS:
            out = impl(_lay(H, lay), M, _lay(S0, lay), lay, d)
            assert np.array_equal(out, _lay(H, lay).astype(np.float64)), (lay, d)


def pin_m_identity(impl, seed=12):
    """M = I: forward gives S0 + prefix sums of H, backward S0 + suffix sums (exact on integers)."""
    n, K, V = 6, 5, 7
    H = qi.small_integers(1000 * seed, (3, n, K, V))
    S0 = qi.small_integers(1000 * seed + 2, (3, K, V))
    M = np.broadcast_to(np.eye(K, dtype=np.float32), (3, n, K, K)).copy()
    prefix = np.cumsum(H.astype(np.int64), axis=1) + S0[:, None].astype(np.int64)
    suffix = np.cumsum(H[:, ::-1].astype(np.int64), axis=1)[:, ::-1] + S0[:, None].astype(np.int64)
    for lay in LAYOUTS:
        for d, want in (("fwd", prefix), ("bwd", suffix)):
            out = impl(_lay(H, lay), M, _lay(S0, lay), lay, d)
            assert np.array_equal(out, _lay(want, lay).astype(np.float64)), (lay, d)
        out = impl(_lay(H, lay), M, None, lay, "fwd")
        assert np.array_equal(out, _lay(np.cumsum(H.astype(np.int64), axis=1), lay)), lay


def pin_scalar_geometric(impl):
    """K = V = 1, constant m, h: S_j = m^(j+1) s0 + h (1 - m^(j+1)) / (1 - m)."""
    n, m, h, s0 = 9, 0.75, 1.5, -2.0
    H = np.full((1, n, 1, 1), h)
    M = np.full((1, n, 1, 1), m)
    S0 = np.full((1, 1, 1), s0)
    want = np.array([m ** (j + 1) * s0 + h * (1 - m ** (j + 1)) / (1 - m) for j in range(n)])
    for lay in LAYOUTS:
        fwd = impl(H, M, S0, lay, "fwd").reshape(n)
        bwd = impl(H, M, S0, lay, "bwd").reshape(n)
        assert np.allclose(fwd, want, rtol=1e-13, atol=0), (lay, fwd, want)
        assert np.allclose(bwd, want[::-1], rtol=1e-13, atol=0), (lay, bwd, want)


def pin_diagonal(impl, seed=13):
    """Diagonal M_j: each entry runs its own scalar recurrence (elementwise, no matmul)."""
    n, K, V = 4, 6, 5
    rng = qi.rng(seed)
    d = rng.standard_normal((2, n, K))
    H = rng.standard_normal((2, n, K, V))
    S0 = rng.standard_normal((2, K, V))
    M = np.zeros((2, n, K, K))
    M[:, :, np.arange(K), np.arange(K)] = d
    for dire in DIRECTIONS:
        want = np.empty_like(H)
        s = S0.copy()
        order = range(n) if dire == "fwd" else range(n - 1, -1, -1)
        for j in order:
            s = d[:, j, :, None] * s + H[:, j]
            want[:, j] = s
        for lay in LAYOUTS:
            out = impl(_lay(H, lay), M, _lay(S0, lay), lay, dire)
            assert np.allclose(_kv(out, lay), want, rtol=1e-14, atol=1e-14), (lay, dire)


# ---------------------------------------------------------- exact brute force
def _fr_matmul(A, B):
    return [[sum((A[i][k] * B[k][j] for k in range(len(B))), Fraction(0))
             for j in range(len(B[0]))] for i in range(len(A))]


def _fr_add(A, B):
    return [[A[i][j] + B[i][j] for j in range(len(A[0]))] for i in range(len(A))]


def _fr_T(A):
    return [list(r) for r in zip(*A)]


def _fr_eye(K):
    return [[Fraction(int(i == j)) for j in range(K)] for i in range(K)]


def _fr(a):
    return [[Fraction(float(x)) for x in row] for row in a]


def unrolled_exact(H, M, S0, direction):
    """Exact rational result of one chain from the unrolled-product form.

    forward : out[j] = (M_j ... M_0) S0 + sum_{t<=j} (M_j ... M_{t+1}) H_t
    backward: out[j] = (M_j^T ... M_{n-1}^T) S0 + sum_{t>=j} (M_j^T ... M_{t-1}^T) H_t
    The operator products are formed first, left to right, then applied: a
    different association from the step-by-step recurrence.
    """
    n, K = len(H), len(M[0])
    Hf = [_fr(h) for h in H]
    Mf = [_fr(m) for m in M]
    S0f = _fr(S0) if S0 is not None else None
    out = []
    for j in range(n):
        ts = range(j + 1) if direction == "fwd" else range(j, n)
        acc = [[Fraction(0)] * len(Hf[0][0]) for _ in range(K)]
        for t in ts:
            P = _fr_eye(K)
            steps = range(j, t, -1) if direction == "fwd" else range(j, t)
            for i in steps:
                P = _fr_matmul(P, Mf[i] if direction == "fwd" else _fr_T(Mf[i]))
            acc = _fr_add(acc, _fr_matmul(P, Hf[t]))
        if S0f is not None:
            P = _fr_eye(K)
            steps = range(j, -1, -1) if direction == "fwd" else range(j, n)
            for i in steps:
                P = _fr_matmul(P, Mf[i] if direction == "fwd" else _fr_T(Mf[i]))
            acc = _fr_add(acc, _fr_matmul(P, S0f))
        out.append(acc)
    return out


def pin_bruteforce_exact(impl, seed=14, trials=6):
    """Tiny dyadic inputs: the implementation equals the exact rational result."""
    rng = qi.rng(seed)
    for trial in range(trials):
        n = int(rng.integers(1, 5))
        K = int(rng.integers(1, 4))
        V = int(rng.integers(1, 4))
        H = rng.integers(-8, 9, (1, n, K, V)) / 4.0
        M = rng.integers(-4, 5, (1, n, K, K)) / 4.0
        S0 = rng.integers(-8, 9, (1, K, V)) / 4.0 if trial % 2 == 0 else None
        for d in DIRECTIONS:
            exact = unrolled_exact(H[0], M[0], None if S0 is None else S0[0], d)
            want = np.array([[[float(x) for x in row] for row in s] for s in exact])
            for lay in LAYOUTS:
                out = impl(_lay(H, lay), M, None if S0 is None else _lay(S0, lay), lay, d)
                assert np.array_equal(_kv(out, lay)[0], want), (trial, lay, d)


def apply_signed_perm(perm, sign, x, transpose):
    """(P x) with P[a, perm[a]] = sign[a], by index moves only (no products)."""
    y = np.empty_like(x)
    if not transpose:
        y[:] = sign[:, None] * x[perm]
    else:
        y[perm] = sign[:, None] * x
    return y


def pin_signed_permutation(impl, seed=15):
    """Signed-permutation M with integer H, S0: exact integer result by index moves."""
    n, K, V = 5, 8, 6
    H = qi.small_integers(1000 * seed, (2, n, K, V))
    S0 = qi.small_integers(1000 * seed + 2, (2, K, V))
    M = qi.signed_permutations(1000 * seed + 1, (2, n), K)
    perms = np.argmax(np.abs(M), axis=-1)
    signs = np.take_along_axis(M, perms[..., None], axis=-1)[..., 0].astype(np.int64)
    for d in DIRECTIONS:
        want = np.empty(H.shape, np.int64)
        for c in range(2):
            s = S0[c].astype(np.int64)
            order = range(n) if d == "fwd" else range(n - 1, -1, -1)
            for j in order:
                s = apply_signed_perm(perms[c, j], signs[c, j], s, d == "bwd") + H[c, j].astype(np.int64)
                want[c, j] = s
        for lay in LAYOUTS:
            out = impl(_lay(H, lay), M, _lay(S0, lay), lay, d)
            assert np.array_equal(out, _lay(want, lay).astype(np.float64)), (lay, d)


# -------------------------------------------------------------- invariants
def pin_layout_transpose(impl, seed=16):
    """vk on transposed inputs equals the transpose of kv (same M)."""
    H, M, S0 = qi.random_case(seed, (2,), 4, 6, 9)
    for d in DIRECTIONS:
        kv = impl(H, M, S0, "kv", d)
        vk = impl(qi.to_vk(H), M, qi.to_vk(S0), "vk", d)
        assert np.allclose(qi.to_vk(vk), kv, rtol=1e-13, atol=1e-13), d


def pin_layout_transpose_square(impl, seed=20):
    """As pin_layout_transpose with K = V and a non-symmetric S0: a vk path that
    reads S0, H or out in the kv orientation (shapes alike) must still fail."""
    H, M, S0 = qi.random_case(seed, (2,), 3, 5, 5)
    assert not np.allclose(S0, np.swapaxes(S0, -1, -2))
    for d in DIRECTIONS:
        kv = impl(H, M, S0, "kv", d)
        vk = impl(qi.to_vk(H), M, qi.to_vk(S0), "vk", d)
        assert np.allclose(qi.to_vk(vk), kv, rtol=1e-13, atol=1e-13), d


def pin_adjoint(impl, seed=17):
    """<fwd_M(X), Y> = <X, bwd_M'(Y)> with S0 = 0 and M'_j = M_{j+1} (M'_{n-1} arbitrary)."""
    n, K, V = 5, 7, 4
    rng = qi.rng(seed)
    X = rng.standard_normal((1, n, K, V))
    Y = rng.standard_normal((1, n, K, V))
    M = rng.standard_normal((1, n, K, K)) / np.sqrt(K)
    Mp = np.concatenate([M[:, 1:], rng.standard_normal((1, 1, K, K))], axis=1)
    for lay in LAYOUTS:
        lhs = np.sum(_kv(impl(_lay(X, lay), M, None, lay, "fwd"), lay) * Y)
        rhs = np.sum(X * _kv(impl(_lay(Y, lay), Mp, None, lay, "bwd"), lay))
        assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(lhs)), (lay, lhs, rhs)


def pin_reverse(impl, seed=18):
    """bwd(H, M, S0)[j] = fwd(reversed H, reversed M^T, S0)[n-1-j]."""
    H, M, S0 = qi.random_case(seed, (2,), 5, 6, 5)
    Mt_rev = np.ascontiguousarray(np.swapaxes(M, -1, -2)[:, ::-1])
    for lay in LAYOUTS:
        bwd = impl(_lay(H, lay), M, _lay(S0, lay), lay, "bwd")
        fwd = impl(_lay(np.ascontiguousarray(H[:, ::-1]), lay), Mt_rev, _lay(S0, lay), lay, "fwd")
        assert np.allclose(bwd, fwd[:, ::-1], rtol=1e-13, atol=1e-13), lay


def pin_linearity(impl, seed=19):
    """out(aH + bH', aS0 + bS0') = a out(H, S0) + b out(H', S0')."""
    H, M, S0 = qi.random_case(seed, (2,), 4, 5, 6)
    H2, _, S02 = qi.random_case(seed + 100, (2,), 4, 5, 6)
    H, S0, H2, S02 = (x.astype(np.float64) for x in (H, S0, H2, S02))
    a, b = 0.75, -1.25
    Hc = a * H + b * H2
    Sc = a * S0 + b * S02
    for lay in LAYOUTS:
        for d in DIRECTIONS:
            lhs = impl(_lay(Hc, lay), M, _lay(Sc, lay), lay, d)
            rhs = a * impl(_lay(H, lay), M, _lay(S0, lay), lay, d) + \
                b * impl(_lay(H2, lay), M, _lay(S02, lay), lay, d)
            assert np.allclose(lhs, rhs, rtol=1e-12, atol=1e-12), (lay, d)


def pin_coded_sentinel(impl):
    """M = 0 with coded H: out equals H bit for bit, so no segment reads another's data."""
    n, K, V = 6, 16, 12
    H = qi.coded_states((2,), n, K, V)
    M = np.zeros((2, n, K, K), np.float32)
    S0 = np.full((2, K, V), 7.0, np.float32)
    for lay in LAYOUTS:
        for d in DIRECTIONS:
            out = impl(_lay(H, lay), M, _lay(S0, lay), lay, d)
            bad = np.argwhere(out != _lay(H, lay))
            assert bad.size == 0, (lay, d, bad[:3])


def pin_golden(impl):
    """Hand-worked 2 x 2 example stored under tests/golden/."""
    with open(os.path.join(GOLDEN_DIR, "handworked_k2_n2.json")) as f:
        g = json.load(f)
    H = np.array(g["H"], np.float64)[None]
    M = np.array(g["M"], np.float64)[None]
    for case in g["cases"]:
        S0 = None if case["S0"] is None else np.array(case["S0"], np.float64)[None]
        want = np.array(case["out"], np.float64)
        for lay in LAYOUTS:
            out = impl(_lay(H, lay), M, None if S0 is None else _lay(S0, lay), lay, case["direction"])
            assert np.array_equal(_kv(out, lay)[0], want), (case["name"], lay)


ALL_PINS = [
    pin_m_zero, pin_m_identity, pin_scalar_geometric, pin_diagonal,
    pin_bruteforce_exact, pin_signed_permutation, pin_layout_transpose, pin_layout_transpose_square,
    pin_adjoint, pin_reverse, pin_linearity, pin_coded_sentinel, pin_golden,
]
