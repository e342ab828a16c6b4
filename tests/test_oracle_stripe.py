"""Pins for the oracle's stripe map and strided KV-cache write reference.

The map is pinned by hand-worked fixtures (tests/golden/stripe_maps.json),
by brute-force counting against the closed-form shard lengths, by the
bijection property of the slot map, and by a bitwise round trip.
"""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_stripe_golden_fixture():
    cases = json.load(open(os.path.join(GOLDEN, "stripe_maps.json")))["cases"]
    for c in cases:
        L, P, I = c["cache_len"], c["P"], c["interleave"]
        lens = oracle.shard_lengths(L, P, I)
        assert lens == [len(s) for s in c["shards"]]
        cap = max(lens + [1])
        ids = np.arange(L, dtype=np.int64)[:, None]
        striped = oracle.stripe(ids, P, I, cap, fill=-1)
        for s, expect in enumerate(c["shards"]):
            assert striped[s, :len(expect), 0].tolist() == expect
            assert (striped[s, len(expect):, 0] == -1).all()


@pytest.mark.parametrize("P", [1, 2, 3, 5, 8])
@pytest.mark.parametrize("I", [1, 2, 3, 16])
def test_shard_lengths_match_counting(P, I):
    for L in list(range(0, 70)) + [126973 % 997, 1000]:
        counts = [0] * P
        slots = [set() for _ in range(P)]
        for p in range(L):
            s, j = oracle.stripe_position(p, P, I)
            counts[s] += 1
            slots[s].add(j)
        assert oracle.shard_lengths(L, P, I) == counts
        # the slot map is a bijection onto [0, len) within each shard
        for s in range(P):
            assert slots[s] == set(range(counts[s]))


def test_config_shard_lengths():
    # 128k irregular context: 126973 = 15871 * 8 + 5 -> five shards one longer
    assert oracle.shard_lengths(126973, 8, 1) == [15872] * 5 + [15871] * 3
    assert oracle.shard_lengths(28672, 8, 1) == [3584] * 8


@pytest.mark.parametrize("P,I", [(1, 1), (2, 1), (3, 2), (8, 1), (4, 64), (7, 3)])
def test_stripe_roundtrip_bitwise(P, I):
    rng = np.random.default_rng(P * 100 + I)
    L = 157
    x = rng.integers(0, 2 ** 16, size=(L, 2, 8), dtype=np.uint16)
    cap = max(oracle.shard_lengths(L, P, I))
    st = oracle.stripe(x, P, I, cap, fill=0xFFFF)
    back = oracle.destripe(st, L, P, I)
    assert back.dtype == np.uint16 and np.array_equal(back, x)


@pytest.mark.parametrize("P,I,L,n", [(2, 1, 512, 128), (8, 1, 28672 % 1000, 96),
                                      (3, 2, 11, 7), (8, 16, 5, 40), (1, 1, 0, 9)])
def test_kv_cache_write_ref(P, I, L, n):
    rng = np.random.default_rng(L + n)
    nkv, hd = 2, 8
    cap = max(oracle.shard_lengths(L + n, P, I) + [1])
    old = rng.integers(0, 2 ** 16, size=(L, nkv, hd), dtype=np.uint16)
    sentinel = 0x7FC1  # a NaN pattern; must survive in untouched slots
    kc = oracle.stripe(old, P, I, cap, fill=sentinel)
    vc = kc.copy()
    kcur = rng.integers(0, 2 ** 16, size=(n, nkv, hd), dtype=np.uint16)
    vcur = rng.integers(0, 2 ** 16, size=(n, nkv, hd), dtype=np.uint16)
    kc2, vc2 = oracle.kv_cache_write_ref(kc, vc, kcur, vcur, n, L, P, I)
    # new tokens land in token order after the old ones
    assert np.array_equal(oracle.destripe(kc2, L + n, P, I), np.concatenate([old, kcur]))
    assert np.array_equal(oracle.destripe(vc2, L + n, P, I), np.concatenate([old, vcur]))
    # slots beyond each shard's new length are untouched
    lens = oracle.shard_lengths(L + n, P, I)
    for s in range(P):
        assert (kc2[s, lens[s]:] == sentinel).all()
        assert (vc2[s, lens[s]:] == sentinel).all()
    # inputs were not modified
    assert np.array_equal(oracle.destripe(kc, L, P, I), old)
