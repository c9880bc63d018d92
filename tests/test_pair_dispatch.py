"""Which plain calls run two tiles per workgroup (no GPU: the forced-delay test
library exports the launcher's decision as qla_test_pairs_tiles).

At K >= 96 one workgroup of either kernel fills a CU's LDS, a call runs in
rounds of one workgroup per CU, and a two-tile workgroup takes 1.7-2.0x as
long as a one-tile one: pairs are chosen when 1.8 x their rounds is below the
single tiles' rounds.  Below K = 96 several workgroups share a CU: pairs above
three tiles per CU (at K = 64 up to four), and at K = 64 also at one to two
tiles per CU for chains of 32 or more segments.  The expected decisions are those the measured
timings favour on 256 CUs (K = 32 to 128, 8 to 64 segments)."""
import ctypes
import os

import pytest

import linear_attention_context_amd as qla


@pytest.fixture(scope="module")
def rule():
    if not os.path.exists(qla.library_path("delay")):
        from linear_attention_context_amd import build
        build.build()
    lib = qla.load_library(qla.library_path("delay"))
    f = lib.qla_test_pairs_tiles
    f.argtypes = [ctypes.c_int, ctypes.c_longlong, ctypes.c_int, ctypes.c_int, ctypes.c_int]
    f.restype = ctypes.c_int
    return lambda K, chains, V, n=8, cus=256: bool(f(K, chains, V, n, cus))


@pytest.mark.parametrize("heads,pairs", [
    (16, False), (32, False),                  # one round of single tiles
    (40, True), (48, True), (56, True), (64, True),  # 1-2 tiles per CU: one round of pairs against two
    (72, False), (80, False), (96, False),     # 2-3 per CU: two rounds of pairs lose to three
    (112, True), (128, True),                  # 3-4 per CU: two against four (the long chain, 4 x 32 heads)
])
@pytest.mark.parametrize("n", [8, 64])
def test_k128_rounds(rule, heads, pairs, n):
    assert rule(128, heads, 128, n) is pairs


@pytest.mark.parametrize("chains,pairs", [(42, False), (43, True), (64, True), (86, False), (128, False),
                                          (171, False), (256, True)])
def test_k96_rounds(rule, chains, pairs):
    # V = 96: six tiles per chain, three pairs
    assert rule(96, chains, 96) is pairs


@pytest.mark.parametrize("chains,n,pairs", [
    (96, 8, False), (128, 8, False), (160, 8, False), (192, 8, False),   # up to 3 tiles per CU
    (193, 8, True), (256, 8, True), (257, 8, False), (384, 8, False),    # 3-4 only
    (64, 32, False), (96, 32, True), (128, 32, True), (129, 32, False),  # long chains: 1-2 per CU too
    (160, 64, False), (256, 64, True),
])
def test_k64(rule, chains, n, pairs):
    # V = 64: four tiles per chain
    assert rule(64, chains, 64, n) is pairs


@pytest.mark.parametrize("chains,n,pairs", [(192, 64, False), (384, 64, False), (385, 64, True), (512, 8, True)])
def test_k32(rule, chains, n, pairs):
    # V = 32: two tiles per chain; no exception for long chains below three tiles per CU
    assert rule(32, chains, 32, n) is pairs


def test_never_for_single_tiles_or_other_k(rule):
    assert not rule(128, 4096, 16)     # one tile per chain
    assert not rule(112, 4096, 128)    # K not a multiple of 32
    assert not rule(256, 4096, 256)    # the general kernel


def test_ragged_v_counts_pairs_per_chain(rule):
    # V = 100: 7 tiles, 4 pairs per chain.  128 chains: 896 tiles (4 rounds),
    # 512 pair workgroups (2 rounds); 129 chains: 516 pair workgroups (3 rounds).
    assert rule(128, 128, 100)
    assert not rule(128, 129, 100)


def test_device_size_enters(rule):
    assert rule(128, 64, 128, cus=256)
    assert not rule(128, 64, 128, cus=512)
    assert rule(64, 256, 64, cus=256) and not rule(64, 256, 64, cus=512)
